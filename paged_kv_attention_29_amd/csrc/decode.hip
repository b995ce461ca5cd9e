// paged_attn_decode: one query token per sequence over the paged KV cache,
// optionally split along the keys (Aphrodite flash_attn.py,
// FlashAttentionImpl.forward, flash_attn_with_kvcache decode; vLLM
// flash_attn.py (e2f56c3), FlashAttentionMetadataBuilder num_splits and its
// intermediate buffers).
//
// Work item = (kv head g, sequence b, split).  Splits are fixed chunks of
// keys sized from the batch bound max_seq_len (vLLM flashinfer.py,
// FlashInferMetadataBuilder, fixed_split_size), so every non-empty work
// item of a batch is about the same size.  The G = Hq / Hkv query heads
// sharing KV head g are the 16 columns of one MFMA tile (padded with zero
// queries; with G > 16 an item takes one group of 16 of them, and with
// G <= 8 one item takes two adjacent KV heads), so each K/V byte is read
// from HBM once for every 16 heads.  Keys
// are processed in tiles of 16 (one MFMA M-tile); block_size is a multiple
// of 16, so a tile never straddles two cache blocks.
//
//   S^T[16 keys x 16 heads] = K_tile[16 x D] . Q^T[D x 16]    (mfma 16x16x32)
//   O^T[D x 16 heads]      += V_tile^T[D x 16] . P^T[16 x 16] (mfma 16x16x16)
//
// K is loaded from HBM straight into the A-operand layout (16-byte pieces of
// a key row per lane).  V needs its key index inside each lane, so each wave
// writes its V tile to a private LDS slab row-major and reads it back with
// the LDS transpose read (one ds_read_b64_tr_b16 per PV MFMA).  The 4 waves
// of a workgroup take interleaved steps of an item with their own
// online-softmax state (fp32, base-2 exponent) and are merged through LDS at
// the item's end.  The loads of a wave's next step are issued before its
// current step is computed.
#include <atomic>
#include <type_traits>

#include "common.h"
#include "launch.h"

namespace pa {

namespace {

constexpr int kWaves = 4;

struct DecodeArgs {
  void* out;
  float* lse;
  float* part_out;
  float* part_lse;
  const uint16_t* q;
  const uint16_t* kc;
  const uint16_t* vc;
  const int32_t* seq_lens;
  const int32_t* block_table;
  int64_t bt_stride;
  int B, Hq, Hkv, G, bs, S;
  // query heads of a KV head beyond 16 are split into column groups of 16:
  // CG groups per KV head (1 when G <= 16), each its own work item
  int CG;
  int chunk;            // keys per split (block-aligned, from the batch bound)
  uint32_t bs_magic;    // ceil(2^32 / bs)
  float scale_log2;     // scale * log2(e)
  float cap_k2;         // 2 log2(e) scale / softcap
  float cap_log2;       // softcap * log2(e)
  int window_left;      // -1 = none
  const float* alibi;   // nullable
  // attention sinks [Hq] (fp32, nullable): one more logit per head in the
  // softmax denominator, without a value; folded into split 0 only
  const float* sinks;
  // fp8 (e4m3) cache: device fp32 scales (the stored codes times the scale
  // are the K / V values); null for a 16-bit cache
  const float* k_scale;
  const float* v_scale;
  // fp8 query (with an fp8 cache): q holds e4m3 codes and this device fp32
  // scalar is their descale; null for a 16-bit query
  const float* q_scale;
  // merged splits (S > 1): one int counter per (sequence, column group),
  // zero on entry and left zero; the last split item of a (sequence, column
  // group) to finish merges the partial results into out / lse.  Null: the
  // partials are the result.
  int* counters;
  // timeline trace records (trace library only), or null
  uint64_t* trace;
};

enum { kSoftcap = 1, kAlibi = 2, kFp8 = 4, kQ8 = 8 };
constexpr float kTau = 8.0f;  // lazy-rescale threshold (log2 units)

// A work item covers HPW adjacent KV heads (2 when the head counts allow it
// and D <= 128): each key row of the item is then 2 * 256 contiguous bytes,
// which the memory system streams faster than 256-byte rows 2 KB apart.
// Their query heads are the first G * HPW columns of the MFMA tile.  With
// more than 16 query heads per KV head (HPW = 1) an item covers one group
// of 16 of them (the last group may be smaller), and the groups of a KV
// head are consecutive items, so the K/V bytes they share are read from
// HBM once and then from the caches.
// Keys per iteration: NT MFMA row tiles of 16, so that a wave keeps 16 KB of
// K/V in flight while it computes the previous step (one tile for two heads
// or D = 256; an fp8 cache at D = 256, whose rows are half as long and
// whose workgroup has the CU to itself, takes two).
template <int D, int HPW, bool F8 = false>
constexpr int kNT = ((D <= 128 && HPW == 1) || (F8 && D == 256)) ? 2 : 1;

// LDS: per-wave V slabs of 16 * NT rows (pitch D + 16 elements: the 32-byte
// pad spreads the 16 rows a transpose read touches over all banks) and the
// cross-wave combine area [wave][head j < G * HPW][m, l, pad, pad, O[D]]
// (fp32).
template <int D, int HPW>
constexpr int kVPitch = HPW * D + 16;
template <int D, int HPW, bool F8>
constexpr size_t vslab_bytes() {
  return (size_t)kWaves * 16 * kNT<D, HPW, F8> * kVPitch<D, HPW> * 2;
}
template <int D, int HPW>
constexpr size_t comb_bytes(int G) {
  const int cols = G * HPW < 16 ? G * HPW : 16;  // columns of one item
  return (size_t)kWaves * cols * (D + 4) * 4;
}
// The combine runs after the key loop and reuses the V slabs.  The
// work-item ranking runs before both (scratch ints at the start, below) and
// hands its result over in a 16-byte slot past the slabs, the combine area
// and the scratch, which nothing else writes.
constexpr size_t kRankScratchBytes = (64 + 1 + 1024) * 4;
template <int D, int HPW, bool F8>
constexpr size_t rank_slot_offset(int G) {
  const size_t vc = vslab_bytes<D, HPW, F8>() > comb_bytes<D, HPW>(G) ? vslab_bytes<D, HPW, F8>()
                                                                       : comb_bytes<D, HPW>(G);
  const size_t m = vc > kRankScratchBytes ? vc : kRankScratchBytes;
  return (m + 15) / 16 * 16;
}
template <int D, int HPW, bool F8>
constexpr size_t decode_lds_bytes(int G) {
  return rank_slot_offset<D, HPW, F8>(G) + 16;
}

template <int D>
constexpr int kMinBlocks = D <= 128 ? 2 : 1;

// Keys [lo, hi) of split p of a sequence of length L, and the first visible
// one (sliding window); the split has work iff lo_vis < hi.
struct SplitRange {
  int lo, hi, lo_vis;
};
__device__ __forceinline__ SplitRange split_range(const DecodeArgs& a, int L, int p) {
  SplitRange r;
  // split p covers keys [p * chunk, (p + 1) * chunk) of the sequence; the
  // last split also takes any keys past S * chunk
  r.lo = static_cast<int>(min((int64_t)p * a.chunk, (int64_t)L));
  r.hi = p == a.S - 1 ? L : min(r.lo + a.chunk, L);
  r.lo_vis = a.window_left >= 0 ? max(r.lo, L - 1 - a.window_left) : r.lo;
  return r;
}

// Splits pf..pl of a sequence of L > 0 keys have visible keys (split_range
// gives lo_vis < hi exactly for these; a zero chunk leaves every key to the
// last split).
__device__ __forceinline__ void split_span(const DecodeArgs& a, int L, int& pf, int& pl) {
  const int lw = a.window_left >= 0 ? max(L - 1 - a.window_left, 0) : 0;
  pf = a.chunk > 0 ? min(lw / a.chunk, a.S - 1) : a.S - 1;
  pl = a.chunk > 0 ? min((L - 1) / a.chunk, a.S - 1) : a.S - 1;
}

// Work-item order for batches of at most kRankMaxB sequences and kRankMaxS
// splits: workgroup i takes the i-th item of the list "every (sequence,
// split) pair with visible keys, split-major, sequences in index order,
// KV-head groups fastest; then the empty pairs in the same order".  Empty
// items only write their zero / -inf result, but each still holds a
// workgroup slot while it waits for its sequence length behind the loads in
// flight; listed last, they run while the last real items finish instead of
// taking slots between them.  Wave 0 of every workgroup derives the order
// from seq_lens (LDS scratch: the per-split difference counts and the
// lengths) and hands the item to the other waves through a slot past the V
// slabs and the combine area, so no pass runs before the kernel.  Other
// batches use the plain split-major order.
constexpr int kRankMaxB = 1024;
constexpr int kRankMaxS = 64;
static_assert((kRankMaxS + 1 + kRankMaxB) * 4 <= kRankScratchBytes, "ranking scratch size");

// wave 0 only; sh = LDS scratch, res = the hand-off slot (4 ints)
template <int HPW>
__device__ void ranked_item_wave0(const DecodeArgs& a, int* sh, int* res) {
  const int S = a.S, B = a.B, HG = a.Hkv / HPW * a.CG;
  const int lane = threadIdx.x & 63;
  int* cnt = sh;                  // [S + 1] difference counts
  int* lens = sh + kRankMaxS + 1; // [B]
  if (lane <= S) cnt[lane] = 0;
  if (lane == 0 && S == 64) cnt[64] = 0;
  wave_lds_sync();
  for (int b0 = 0; b0 < B; b0 += 64) {
    const int b = b0 + lane;
    if (b < B) {
      const int L = a.seq_lens[b];
      lens[b] = L;
      if (L > 0) {
        int pf, pl;
        split_span(a, L, pf, pl);
        atomicAdd(cnt + pf, 1);
        atomicAdd(cnt + pl + 1, -1);
      }
    }
  }
  wave_lds_sync();  // the adds of every lane land before the reads
  const int d = lane < S ? cnt[lane] : 0;
  // lane p: c = sequences with a non-empty split p, base = non-empty pairs
  // of the splits before p
  int run_c = 0, run_b = 0, base = 0;
  for (int p = 0; p < S; ++p) {
    run_c += __builtin_amdgcn_readlane(d, p);
    base = lane == p ? run_b : base;
    run_b += run_c;
  }
  const int total = run_b;
  int idx = static_cast<int>(blockIdx.x);
  const bool want = idx < total * HG;  // a non-empty item
  if (!want) idx -= total * HG;
  const int r = idx / HG;
  const int g = idx - r * HG;
  // the split: the last p whose list of items starts at or before r (the
  // starts grow with p, so those p are a prefix of the lanes)
  const int start = want ? base : lane * B - base;
  const uint64_t before = __builtin_amdgcn_ballot_w64(lane < S && start <= r);
  const int split = static_cast<int>(__builtin_popcountll(before)) - 1;
  int rr = r - __builtin_amdgcn_readlane(start, split);
  // the rr-th sequence, in index order, whose split is (non-)empty
  int sel = -1;
  for (int b0 = 0; b0 < B; b0 += 64) {
    const int b = b0 + lane;
    bool flag = false;
    if (b < B) {
      const int L = lens[b];
      bool ne = false;
      if (L > 0) {
        int pf, pl;
        split_span(a, L, pf, pl);
        ne = pf <= split && split <= pl;
      }
      flag = ne == want;
    }
    const uint64_t m = __builtin_amdgcn_ballot_w64(flag);
    const int n = static_cast<int>(__builtin_popcountll(m));
    if (rr < n) {
      const int rank = static_cast<int>(__builtin_popcountll(m & ((1ull << lane) - 1)));
      const uint64_t hit = __builtin_amdgcn_ballot_w64(flag && rank == rr);
      sel = b0 + static_cast<int>(__builtin_ctzll(hit));
      break;
    }
    rr -= n;
  }
  // (every workgroup finds its item, since the grid holds exactly HG * B * S
  // of them; sel < 0 would mean inconsistent lengths and makes the kernel
  // exit)
  if (lane == 0) {
    res[0] = g;
    res[1] = sel;
    res[2] = split;
    res[3] = sel >= 0 ? lens[sel] : 0;
  }
}

// The pieces of one work item.
template <typename T, int D, int FEAT, int HPW>
struct Dec {
  using TT = T;
  static constexpr int kD = D;
  static constexpr int kHPW = HPW;
  static constexpr bool SOFTCAP = FEAT & kSoftcap;
  static constexpr bool ALIBI = FEAT & kAlibi;
  static constexpr bool F8 = FEAT & kFp8;
  static constexpr bool Q8 = FEAT & kQ8;  // fp8 query codes (widened exactly to T)
  static constexpr int KK = D / 32;   // QK mfma steps along D
  static constexpr int NU = D / 64;   // fp8: 16-byte pieces of a row per lane
  static constexpr int DC = D / 16;   // PV output chunks of 16 rows of D
  static constexpr int NT = kNT<D, HPW, F8>;
  static constexpr int KPS = 16 * NT; // keys per step
  static constexpr int P = kVPitch<D, HPW>;
  static constexpr int CP = D + 4;    // combine row: m, l, 2 pad, O[D] (16-byte aligned)

  // 16-bit cache: lane (r16, c4) holds elements kk*32 + 8*c4 + [0, 8) of
  // key row r16 for each QK step kk.  fp8 cache: it holds bytes
  // u*64 + 16*c4 + [0, 16) (16-byte loads, half the bytes); QK step kk then
  // contracts elements (kk/2)*64 + 16*c4 + 8*(kk%2) + [0, 8), and load_q
  // takes Q in the same order (a permutation of the sum over d).
  struct Frag16 {
    v8s k[HPW][NT][KK];
    v8s v[HPW][NT][KK];
  };
  struct Frag8 {
    u32x4 k[HPW][NT][NU];
    u32x4 v[HPW][NT][NU];
  };
  using Frag = std::conditional_t<F8, Frag8, Frag16>;
  // element offset of this lane's 8 Q / K elements of QK step kk
  static __device__ __forceinline__ int qk_off(int kk, int c4) {
    return F8 ? (kk >> 1) * 64 + 16 * c4 + 8 * (kk & 1) : kk * 32 + 8 * c4;
  }
  // the 16-bit K operand of QK step kk
  static __device__ __forceinline__ v8s k_operand(const Frag& f, int h, int nt, int kk) {
    if constexpr (F8) {
      const u32x4& w = f.k[h][nt][kk >> 1];
      const v4s lo = T::from_fp8x4(w[2 * (kk & 1)]);
      const v4s hi = T::from_fp8x4(w[2 * (kk & 1) + 1]);
      return v8s{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    } else {
      return f.k[h][nt][kk];
    }
  }

  // KV heads g0 .. g0 + HPW - 1 of sequence b, keys [lo_vis, hi) of `split`;
  // its columns are query heads hb .. hb + nc - 1
  struct Item {
    int g0, b, split;
    int hb, nc;
    int pos;             // the query's position, L - 1
    int lo_vis, hi;
    int s_begin, s_end;  // steps of KPS keys that cover [lo_vis, hi)
    int last_j0;         // first key of the split's last tile of 16
  };

  // grp: the item's column group, (KV head group) * CG + (group of 16)
  static __device__ __forceinline__ Item make_item(const DecodeArgs& a, int grp, int b,
                                                   int split, int L) {
    Item it;
    const int kvg = grp / a.CG;
    const int cg = grp - kvg * a.CG;
    it.g0 = kvg * HPW;
    it.hb = it.g0 * a.G + 16 * cg;
    it.nc = HPW == 2 ? 2 * a.G : min(16, a.G - 16 * cg);
    it.b = b;
    it.split = split;
    it.pos = L - 1;
    const SplitRange r = split_range(a, L, split);
    it.lo_vis = r.lo_vis;
    it.hi = r.hi;
    it.s_begin = r.lo_vis / KPS;
    it.s_end = (r.hi + KPS - 1) / KPS;
    it.last_j0 = r.hi > 0 ? ((r.hi - 1) & ~15) : 0;
    return it;
  }

  // Block ids of a step's tiles.  Loads are branch-free (so the compiler can
  // count outstanding loads exactly): a tile starting at or past hi is
  // clamped to the split's last tile, loaded, and fully masked.  The clamped
  // tile starts before hi, so it lies inside the sequence's last used block
  // at worst (block_size is a multiple of 16) and its block-table entry is
  // valid.
  static __device__ __forceinline__ int tile_j0(const Item& it, int step, int nt) {
    return min(step * KPS + 16 * nt, it.last_j0);
  }
  static __device__ __forceinline__ void fetch_ids(const DecodeArgs& a, const Item& it, int step,
                                                   int (&ids)[NT]) {
    const int32_t* btab = a.block_table + (int64_t)it.b * a.bt_stride;
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) ids[nt] = btab[div_magic(tile_j0(it, step, nt), a.bs_magic)];
  }
  static __device__ __forceinline__ void load_step(const DecodeArgs& a, const Item& it, int step,
                                                   const int (&ids)[NT], int r16, int c4,
                                                   Frag& f) {
    const int64_t row_stride = (int64_t)a.Hkv * D;  // elements between consecutive slots
    if constexpr (F8) {
      const uint8_t* kcg = reinterpret_cast<const uint8_t*>(a.kc) + (int64_t)it.g0 * D + c4 * 16;
      const uint8_t* vcg = reinterpret_cast<const uint8_t*>(a.vc) + (int64_t)it.g0 * D + c4 * 16;
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        const int j0 = tile_j0(it, step, nt);
        const int q = div_magic(j0, a.bs_magic);
        const int64_t slot = (int64_t)ids[nt] * a.bs + (j0 - q * a.bs) + r16;
        const uint8_t* kp = kcg + slot * row_stride;
        const uint8_t* vp = vcg + slot * row_stride;
#pragma unroll
        for (int h = 0; h < HPW; ++h)
#pragma unroll
          for (int u = 0; u < NU; ++u) {
            f.k[h][nt][u] = *reinterpret_cast<const u32x4*>(kp + h * D + u * 64);
            f.v[h][nt][u] = *reinterpret_cast<const u32x4*>(vp + h * D + u * 64);
          }
      }
      return;
    } else {
    const uint16_t* kcg = a.kc + (int64_t)it.g0 * D + c4 * 8;
    const uint16_t* vcg = a.vc + (int64_t)it.g0 * D + c4 * 8;
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      const int j0 = tile_j0(it, step, nt);
      const int q = div_magic(j0, a.bs_magic);
      const int64_t slot = (int64_t)ids[nt] * a.bs + (j0 - q * a.bs) + r16;
      const uint16_t* kp = kcg + slot * row_stride;
      const uint16_t* vp = vcg + slot * row_stride;
#pragma unroll
      for (int h = 0; h < HPW; ++h)
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) {
          f.k[h][nt][kk] = *reinterpret_cast<const v8s*>(kp + h * D + kk * 32);
          f.v[h][nt][kk] = *reinterpret_cast<const v8s*>(vp + h * D + kk * 32);
        }
    }
    }
  }

  // The Q row of this lane's column (head g0 * G + r16; padding columns load
  // the item's first head and are masked by mask_q), without a branch.  An
  // fp8 query is loaded as its codes (8 bytes per step) and widened in
  // mask_q, after the wait for the first K/V step.
  using QRaw = std::conditional_t<Q8, u32x2, v8s>;
  static __device__ __forceinline__ void load_q(const DecodeArgs& a, const Item& it, int r16,
                                                int c4, QRaw (&qraw)[KK]) {
    const int hq = it.hb + (r16 < it.nc ? r16 : 0);
    if constexpr (Q8) {
      const uint8_t* qrow = reinterpret_cast<const uint8_t*>(a.q) + ((int64_t)it.b * a.Hq + hq) * D;
#pragma unroll
      for (int kk = 0; kk < KK; ++kk) qraw[kk] = *reinterpret_cast<const u32x2*>(qrow + qk_off(kk, c4));
    } else {
      const uint16_t* qrow = a.q + ((int64_t)it.b * a.Hq + hq) * D;
#pragma unroll
      for (int kk = 0; kk < KK; ++kk) qraw[kk] = *reinterpret_cast<const v8s*>(qrow + qk_off(kk, c4));
    }
  }
  static __device__ __forceinline__ v8s q_elems(const QRaw& r) {
    if constexpr (Q8) {
      const v4s lo = T::from_fp8x4(r[0]), hi = T::from_fp8x4(r[1]);
      return v8s{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    } else {
      return r;
    }
  }
  // Q^T as the B operand: column r16, D elements kk*32 + c4*8 .. +8; with two
  // KV heads, operand h is zero outside head h's columns, so the two products
  // accumulate into one S^T tile
  static __device__ __forceinline__ void mask_q(const QRaw (&qraw)[KK], bool col_ok, int hsel,
                                                v8s (&qf)[HPW][KK]) {
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
      const v8s z = {0, 0, 0, 0, 0, 0, 0, 0};
      const v8s qv = q_elems(qraw[kk]);
#pragma unroll
      for (int h = 0; h < HPW; ++h) qf[h][kk] = (col_ok && hsel == h) ? qv : z;
    }
  }
  // ALiBi slope of this lane's column, in log2 units
  static __device__ __forceinline__ float slope_of(const DecodeArgs& a, const Item& it, int r16) {
    if constexpr (ALIBI)
      return r16 < it.nc ? a.alibi[it.hb + r16] * kLog2e : 0.0f;
    else
      return 0.0f;
  }

  // One step of KPS keys: scores, online softmax, P.V.  m_run is the
  // reference max (log2 units) of column r16, l_run this lane's share of the
  // running sum, o the lane's O^T[d = dc*16 + 4*c4 + e][head r16].
  static __device__ __forceinline__ void compute_step(const DecodeArgs& a, const Item& it,
                                                      int step, const Frag& f,
                                                      const v8s (&qf)[HPW][KK], float slope_log2,
                                                      int r16, int c4, int hsel, uint16_t* vs,
                                                      float& m_run, float& l_run, v4f (&o)[DC]) {
    float x[NT][4];
    float mx = kNegInf;
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      const int j0 = step * KPS + 16 * nt;
      // ---- scores S^T[key j0 + 4*c4 + e][head r16], in log2 units
      v4f sc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int h = 0; h < HPW; ++h)
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) sc = T::mfma16x16x32(k_operand(f, h, nt, kk), qf[h][kk], sc);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int key = j0 + 4 * c4 + e;
        float v;
        if constexpr (SOFTCAP) v = softcap_log2(sc[e], a.cap_k2, a.cap_log2);
        else v = sc[e] * a.scale_log2;
        if constexpr (ALIBI) v -= slope_log2 * static_cast<float>(it.pos - key);
        x[nt][e] = (key >= it.lo_vis && key < it.hi) ? v : kNegInf;
        mx = fmaxf(mx, x[nt][e]);
      }
    }
    // ---- online softmax per head column; the reference max only moves when
    //      it grows by more than 2^8
    mx = fmaxf(mx, shfl_xor(mx, 16));
    mx = fmaxf(mx, shfl_xor(mx, 32));
    const bool grow = mx > m_run + kTau;
    if (wave_any(grow)) {
      const float m_new = grow ? mx : m_run;
      const float alpha = grow ? fast_exp2(m_run - m_new) : 1.0f;  // 0 when m_run = -inf
      l_run *= alpha;
      // columns whose reference is still -inf hold zeros (no key seen yet)
      if (wave_any(grow && m_run != kNegInf)) {
#pragma unroll
        for (int dc = 0; dc < DC; ++dc) o[dc] *= alpha;
      }
      m_run = m_new;
    }
    const float m_use = m_run == kNegInf ? 0.0f : m_run;
    // P^T as the PV B operand: lane (head r16, quarter c4) holds keys
    // 16*nt + 4*c4 + e of each tile; with two tiles they form one 8-element
    // operand of a 16x16x32 MFMA (key slots 4*c4 + e and 16 + 4*c4 + e)
    uint32_t pw[2 * NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      float pe[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) pe[e] = fast_exp2(x[nt][e] - m_use);
      l_run += (pe[0] + pe[1]) + (pe[2] + pe[3]);
      pw[2 * nt] = T::pack2(pe[0], pe[1]);
      pw[2 * nt + 1] = T::pack2(pe[2], pe[3]);
    }
    // ---- V -> LDS rows 16*nt + r16; rows outside [lo_vis, hi) become zero
    //      so stale or poisoned cache contents never reach the accumulator
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      const int key = step * KPS + 16 * nt + r16;
      const bool row_ok = key >= it.lo_vis && key < it.hi;
      const v8s z = {0, 0, 0, 0, 0, 0, 0, 0};
      if constexpr (F8) {
        // the row's bytes u*64 + 16*c4 + [0, 16) become elements at the same
        // positions of the LDS row
        uint16_t* dst = vs + (16 * nt + r16) * P + c4 * 16;
#pragma unroll
        for (int h = 0; h < HPW; ++h)
#pragma unroll
          for (int u = 0; u < NU; ++u) {
            const u32x4& w = f.v[h][nt][u];
            const v4s e0 = T::from_fp8x4(w[0]), e1 = T::from_fp8x4(w[1]);
            const v4s e2 = T::from_fp8x4(w[2]), e3 = T::from_fp8x4(w[3]);
            const v8s lo = {e0[0], e0[1], e0[2], e0[3], e1[0], e1[1], e1[2], e1[3]};
            const v8s hi = {e2[0], e2[1], e2[2], e2[3], e3[0], e3[1], e3[2], e3[3]};
            *reinterpret_cast<v8s*>(dst + h * D + u * 64) = row_ok ? lo : z;
            *reinterpret_cast<v8s*>(dst + h * D + u * 64 + 8) = row_ok ? hi : z;
          }
      } else {
        uint16_t* dst = vs + (16 * nt + r16) * P + c4 * 8;
#pragma unroll
        for (int h = 0; h < HPW; ++h)
#pragma unroll
          for (int kk = 0; kk < KK; ++kk)
            *reinterpret_cast<v8s*>(dst + h * D + kk * 32) = row_ok ? f.v[h][nt][kk] : z;
      }
    }
    wave_lds_sync();
    // ---- O^T[d][head] += V^T[d][key] P^T[key][head]; lane group c4 reads
    //      V[16*nt + 4*c4 + e][dc*16 + r16] for e = 0..3 with one transpose
    //      read per tile
    const uint16_t* vb = vs + (4 * c4 + (r16 >> 2)) * P + 4 * (r16 & 3);
    if constexpr (NT == 2) {
      const u32x4 pq = {pw[0], pw[1], pw[2], pw[3]};
      const v8s pb = __builtin_bit_cast(v8s, pq);
#pragma unroll
      for (int dc = 0; dc < DC; ++dc) {
        const v4s v0 = lds_read_tr16(vb + dc * 16);
        const v4s v1 = lds_read_tr16(vb + 16 * P + dc * 16);
        const v8s av = {v0[0], v0[1], v0[2], v0[3], v1[0], v1[1], v1[2], v1[3]};
        o[dc] = T::mfma16x16x32(av, pb, o[dc]);
      }
    } else {
      const u32x2 pq = {pw[0], pw[1]};
      const v4s pb = __builtin_bit_cast(v4s, pq);
      // with two KV heads, P is split by column: head h's V only meets the
      // probabilities of head h's columns
      const v4s z = {0, 0, 0, 0};
#pragma unroll
      for (int h = 0; h < HPW; ++h) {
        const v4s pbh = (HPW == 1 || hsel == h) ? pb : z;
#pragma unroll
        for (int dc = 0; dc < DC; ++dc)
          o[dc] = T::mfma16x16x16(lds_read_tr16(vb + h * D + dc * 16), pbh, o[dc]);
      }
    }
    wave_lds_sync();
  }

  // Result of column j (query head hb + j), elements d .. d + 3.
  static __device__ __forceinline__ void emit4(const DecodeArgs& a, int hb, int b, int split,
                                               int j, int d, v4f val, float lse) {
    const int h = hb + j;
    if (a.S > 1 && a.counters != nullptr) {
      // merged splits: device-coherent stores (another XCD's workgroup may
      // merge them), so no L2-wide write-back is needed before the count
      float* po = a.part_out + (((int64_t)split * a.B + b) * a.Hq + h) * D + d;
#pragma unroll
      for (int e = 0; e < 4; ++e) __hip_atomic_store(po + e, val[e], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if (d == 0)
        __hip_atomic_store(a.part_lse + ((int64_t)split * a.Hq + h) * a.B + b, lse, __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
    } else if (a.S > 1) {
      *reinterpret_cast<v4f*>(a.part_out + (((int64_t)split * a.B + b) * a.Hq + h) * D + d) = val;
      if (d == 0) a.part_lse[((int64_t)split * a.Hq + h) * a.B + b] = lse;
    } else {
      const u32x2 w = {T::pack2(val[0], val[1]), T::pack2(val[2], val[3])};
      *reinterpret_cast<u32x2*>(static_cast<uint16_t*>(a.out) + ((int64_t)b * a.Hq + h) * D + d) = w;
      if (d == 0 && a.lse != nullptr) a.lse[(int64_t)h * a.B + b] = lse;
    }
  }
  // Sink logit of column j in log2 units, or -inf (no sinks, or a split
  // other than 0).
  static __device__ __forceinline__ float sink_of(const DecodeArgs& a, int hb, int split, int j) {
    return a.sinks != nullptr && split == 0 ? a.sinks[hb + j] * kLog2e : kNegInf;
  }
  // An item without visible keys: zero output, log-sum-exp -inf (or the
  // sink in split 0).
  static __device__ __forceinline__ void emit_empty(const DecodeArgs& a, const Item& it) {
    for (int idx = threadIdx.x; idx < it.nc * (D / 4); idx += kWaves * 64) {
      const int j = idx / (D / 4);
      emit4(a, it.hb, it.b, it.split, j, (idx - j * (D / 4)) * 4, v4f{0.f, 0.f, 0.f, 0.f},
            sink_of(a, it.hb, it.split, j) * kLn2);
    }
  }

  // Merge the waves' states of an item through LDS (comb) and write its
  // result.  Starts with a barrier: every wave is done with the item (and
  // with its V slab, which comb may reuse) and with the previous item's
  // combine.
  static __device__ __forceinline__ void combine_emit(const DecodeArgs& a, const Item& it,
                                                      int wave, int r16, int c4, float m_run,
                                                      float l_run, const v4f (&o)[DC],
                                                      float* comb) {
    const int GC = it.nc;
    float l_tot = l_run + shfl_xor(l_run, 16);
    l_tot += shfl_xor(l_tot, 32);
    __syncthreads();
    if (r16 < GC) {
      float* row = comb + (wave * GC + r16) * CP;
      if (c4 == 0) *reinterpret_cast<f2*>(row) = f2{m_run, l_tot};
#pragma unroll
      for (int dc = 0; dc < DC; ++dc) *reinterpret_cast<v4f*>(row + 4 + dc * 16 + 4 * c4) = o[dc];
    }
    __syncthreads();
    // four consecutive elements per thread and pass
    for (int idx = threadIdx.x; idx < GC * (D / 4); idx += kWaves * 64) {
      const int j = idx / (D / 4);
      const int d = (idx - j * (D / 4)) * 4;
      f2 ml[kWaves];
      const float sk = sink_of(a, it.hb, it.split, j);  // (max sk, sum 1, output 0)
      float M = sk;
#pragma unroll
      for (int w = 0; w < kWaves; ++w) {
        ml[w] = *reinterpret_cast<const f2*>(comb + (w * GC + j) * CP);
        M = fmaxf(M, ml[w][0]);
      }
      v4f num = {0.f, 0.f, 0.f, 0.f};
      float den = 0.f;
      if (M != kNegInf) {
        den = fast_exp2(sk - M);  // 0 without a sink
#pragma unroll
        for (int w = 0; w < kWaves; ++w) {
          const float fw = fast_exp2(ml[w][0] - M);
          den += fw * ml[w][1];
          num += fw * *reinterpret_cast<const v4f*>(comb + (w * GC + j) * CP + 4 + d);
        }
      }
      // (an fp8 cache's V scale multiplies the result)
      const float inv = den > 0.f ? (F8 ? *a.v_scale : 1.0f) / den : 0.f;
      const float lse = den > 0.f ? (M + __log2f(den)) * kLn2 : kNegInf;
      emit4(a, it.hb, it.b, it.split, j, d, num * inv, lse);
    }
  }
};

// ---------------------------------------------------------------------------
// Merged splits.  A split item's partial result goes to part_out / part_lse
// as without merging; then the item counts itself in its (sequence, column
// group) counter, and the item that brings the count to the number of
// partials the group has merges them all into out / lse and resets the
// counter.  The partials of a group are those of its splits with visible
// keys, plus split 0's when it has none but holds the sinks (its partial is
// the sink alone); a sequence with neither has its zero / -inf result
// written by split 0 directly.  The merge is merge_attn_states's arithmetic
// in its order (parts 0, 1, ...), the absent parts weighing 0.
template <typename K>
__device__ __forceinline__ void merged_tail(const DecodeArgs& a, const typename K::Item& it,
                                            int grp, int L, bool wrote, int* flag) {
  constexpr int D = K::kD;
  const bool sinks = a.sinks != nullptr;
  int pf = 0, pl = -1;  // splits with visible keys
  if (L > 0) split_span(a, L, pf, pl);
  const bool sink_part = sinks && (L <= 0 || pf > 0);  // split 0: the sink alone
  const int parts = (pl - pf + 1) + (sink_part ? 1 : 0);
  auto written = [&](int p) { return (p >= pf && p <= pl) || (p == 0 && sink_part); };
  const int64_t B = a.B;
  if (parts == 0) {
    // no partial at all: split 0 writes the empty result
    if (it.split != 0) return;
    for (int idx = threadIdx.x; idx < it.nc * (D / 4); idx += kWaves * 64) {
      const int j = idx / (D / 4);
      const int d = (idx - j * (D / 4)) * 4;
      const int h = it.hb + j;
      uint16_t* o = static_cast<uint16_t*>(a.out) + ((int64_t)it.b * a.Hq + h) * D + d;
      *reinterpret_cast<u32x2*>(o) = u32x2{0u, 0u};
      if (d == 0 && a.lse != nullptr) a.lse[(int64_t)h * B + it.b] = kNegInf;
    }
    return;
  }
  if (!wrote) return;
  // The partials were stored device-coherent (emit4); waiting for them here
  // puts them at the device's coherence point before the count.  (A fence
  // at agent scope would write back and invalidate the whole L2 of the
  // XCD, for every item.)
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  int* cnt = a.counters + (int64_t)it.b * (a.Hkv / K::kHPW * a.CG) + grp;
  if (threadIdx.x == 0) {
    const int old = __hip_atomic_fetch_add(cnt, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const bool last = old == parts - 1;
    if (last) __hip_atomic_store(cnt, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    *flag = last;
  }
  __syncthreads();
  if (!*flag) return;
  // the other items' partials: device-coherent loads, issued after the
  // count showed that every one of them was stored
  for (int idx = threadIdx.x; idx < it.nc * (D / 4); idx += kWaves * 64) {
    const int j = idx / (D / 4);
    const int d = (idx - j * (D / 4)) * 4;
    const int h = it.hb + j;
    // parts in batches of 8 whose loads go out together (device-coherent
    // loads: issued after the count showed every part stored)
    constexpr int NB = 8;
    float l[NB];
    v4f x[NB];
    auto load_batch = [&](int p0, bool rows) {
#pragma unroll
      for (int i = 0; i < NB; ++i) {
        const int p = p0 + i;
        const bool ok = p < a.S && written(p);
        l[i] = ok ? __hip_atomic_load(a.part_lse + ((int64_t)p * a.Hq + h) * B + it.b,
                                      __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)
                  : kNegInf;
        if (rows) {
          const float* px = a.part_out + (((int64_t)p * B + it.b) * a.Hq + h) * D + d;
#pragma unroll
          for (int e = 0; e < 4; ++e)
            x[i][e] = ok ? __hip_atomic_load(px + e, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) : 0.f;
        }
      }
    };
    // the maximum log-sum-exp (with at most 8 parts the first batch's rows
    // are loaded along with it and kept)
    float m = kNegInf;
    for (int p0 = 0; p0 < a.S; p0 += NB) {
      load_batch(p0, a.S <= NB);
#pragma unroll
      for (int i = 0; i < NB; ++i) m = fmaxf(m, l[i]);
    }
    uint16_t* o = static_cast<uint16_t*>(a.out) + ((int64_t)it.b * a.Hq + h) * D + d;
    if (m == kNegInf) {
      *reinterpret_cast<u32x2*>(o) = u32x2{0u, 0u};
      if (d == 0 && a.lse != nullptr) a.lse[(int64_t)h * B + it.b] = kNegInf;
      continue;
    }
    v4f acc = {0.f, 0.f, 0.f, 0.f};
    float wsum = 0.f;
    for (int p0 = 0; p0 < a.S; p0 += NB) {
      if (a.S > NB) load_batch(p0, true);
#pragma unroll
      for (int i = 0; i < NB; ++i) {
        // parts in order; an absent part weighs 0
        const float w = l[i] == kNegInf ? 0.f : fast_exp2((l[i] - m) * kLog2e);
        wsum += w;
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[e] = w != 0.0f ? __builtin_fmaf(w, x[i][e], acc[e]) : acc[e];
      }
    }
    const float inv = 1.0f / wsum;
    const uint32_t lo = K::TT::from_float(acc[0] * inv) | static_cast<uint32_t>(K::TT::from_float(acc[1] * inv)) << 16;
    const uint32_t hi = K::TT::from_float(acc[2] * inv) | static_cast<uint32_t>(K::TT::from_float(acc[3] * inv)) << 16;
    *reinterpret_cast<u32x2*>(o) = u32x2{lo, hi};
    if (d == 0 && a.lse != nullptr) a.lse[(int64_t)h * B + it.b] = m + __logf(wsum);
  }
}

// ---------------------------------------------------------------------------
// One work item per workgroup.
// Item order: split-major; within split p the (KV-head group, sequence) pairs
// are rotated by p groups.  Workgroup i runs on XCD i % 8 and, within it, on
// the shader engines in turn, so without the rotation all splits of a
// sequence would land on the same XCDs and engines and long sequences would
// load some of them more than others.
template <typename T, int D, int FEAT, int HPW>
__global__ __launch_bounds__(kWaves * 64, kMinBlocks<D>) void decode_kernel(DecodeArgs a) {
  using K = Dec<T, D, FEAT, HPW>;
  extern __shared__ __attribute__((aligned(16))) char smem[];
  const uint64_t t_entry = kTrace ? trace_clock() : 0;
  const uint64_t r_entry = kTrace ? trace_realclock() : 0;
  if constexpr (K::F8) {
    // the K scale multiplies every score
    const float ks = *a.k_scale;
    a.scale_log2 *= ks;
    a.cap_k2 *= ks;
  }
  if constexpr (K::Q8) {
    // and so does an fp8 query's descale
    const float qs = *a.q_scale;
    a.scale_log2 *= qs;
    a.cap_k2 *= qs;
  }

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int r16 = lane & 15;   // key row of the K piece / head column of the tile
  const int c4 = lane >> 4;    // which quarter: keys 4*c4..4*c4+3 of S^T, D piece of K

  int grp, b, split, L;  // column group, sequence, split, length
  if (a.B <= kRankMaxB && a.S <= kRankMaxS) {
    int* res = reinterpret_cast<int*>(smem + rank_slot_offset<D, HPW, K::F8>(a.G));
    if (wave == 0) ranked_item_wave0<HPW>(a, reinterpret_cast<int*>(smem), res);
    __syncthreads();
    grp = __builtin_amdgcn_readfirstlane(res[0]);
    b = __builtin_amdgcn_readfirstlane(res[1]);
    split = __builtin_amdgcn_readfirstlane(res[2]);
    L = __builtin_amdgcn_readfirstlane(res[3]);
    if (b < 0) return;
  } else {
    const int HG = a.Hkv / HPW * a.CG;
    const int per_split = HG * a.B;
    split = blockIdx.x / per_split;
    int j = blockIdx.x - split * per_split - static_cast<int>((int64_t)split * HG % per_split);
    if (j < 0) j += per_split;
    grp = j % HG;
    b = j / HG;
    L = a.seq_lens[b];
  }

  const typename K::Item it = K::make_item(a, grp, b, split, L);
  int* const flag = reinterpret_cast<int*>(smem + rank_slot_offset<D, HPW, K::F8>(a.G));
  if constexpr (kTrace) {
    if (wave == 0) {
      trace_put(a.trace, kTrEntry, t_entry);
      trace_put(a.trace, kTrRealEntry, r_entry);
      trace_put(a.trace, kTrItem, trace_clock());
      trace_put(a.trace, kTrUnits,
                static_cast<uint64_t>(it.lo_vis < it.hi ? max(it.s_end - it.s_begin, 0) : 0));
      trace_put(a.trace, kTrWho, (uint64_t)b << 32 | static_cast<uint32_t>(split));
      trace_hw(a.trace);
    }
  }
  if (it.lo_vis >= it.hi) {
    // (merged: only split 0 of a group holding the sinks writes a partial)
    const bool write = a.counters == nullptr || (split == 0 && a.sinks != nullptr);
    if (write) K::emit_empty(a, it);
    if (a.counters != nullptr) merged_tail<K>(a, it, grp, L, write, flag);
    if constexpr (kTrace) {
      if (wave == 0) trace_put(a.trace, kTrEnd, trace_clock());
    }
    return;
  }
  const bool col_ok = r16 < it.nc;
  const int hsel = r16 / a.G;  // which of the item's KV heads the column reads
  const float slope_log2 = K::slope_of(a, it, r16);

  typename K::QRaw qraw[K::KK];
  K::load_q(a, it, r16, c4, qraw);

  float m_run = kNegInf;
  float l_run = 0.0f;
  v4f o[K::DC];
#pragma unroll
  for (int dc = 0; dc < K::DC; ++dc) o[dc] = v4f{0.f, 0.f, 0.f, 0.f};
  uint16_t* vs = reinterpret_cast<uint16_t*>(smem) + wave * K::KPS * K::P;

  // ---- double buffer: the next step's loads are in flight while the
  //      current one is computed.  Block ids run one step further ahead and
  //      are issued before the K/V loads, so waiting for them never waits for
  //      K/V data (the vector-memory counter completes in issue order).
  typename K::Frag cur, nxt;
  int ids[K::NT];
  int step = it.s_begin + wave;
  if (step < it.s_end) {
    K::fetch_ids(a, it, step, ids);
    K::load_step(a, it, step, ids, r16, c4, cur);
    K::fetch_ids(a, it, min(step + kWaves, it.s_end - 1), ids);
  }
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): Q and the first step landed
  if constexpr (kTrace) {
    if (wave == 0) trace_put(a.trace, kTrLoop0, trace_clock());
  }
  v8s qf[HPW][K::KK];
  K::mask_q(qraw, col_ok, hsel, qf);
  for (; step < it.s_end; step += kWaves) {
    if (step + kWaves < it.s_end) {
      int ids2[K::NT];
      K::fetch_ids(a, it, min(step + 2 * kWaves, it.s_end - 1), ids2);
      K::load_step(a, it, step + kWaves, ids, r16, c4, nxt);
#pragma unroll
      for (int nt = 0; nt < K::NT; ++nt) ids[nt] = ids2[nt];
    }
    K::compute_step(a, it, step, cur, qf, slope_log2, r16, c4, hsel, vs, m_run, l_run, o);
    cur = nxt;
  }
  if constexpr (kTrace) {
    if (wave == 0) trace_put(a.trace, kTrLoop1, trace_clock());
  }
  K::combine_emit(a, it, wave, r16, c4, m_run, l_run, o, reinterpret_cast<float*>(smem));
  if (a.counters != nullptr) merged_tail<K>(a, it, grp, L, true, flag);
  if constexpr (kTrace) {
    const uint64_t t_end = trace_clock();
    if (wave == 0) {
      trace_put(a.trace, kTrEnd, t_end);
      trace_put(a.trace, kTrRealEnd, trace_realclock());
    }
    trace_put(a.trace, kTrWaveEnd + wave, t_end);
  }
}

template <typename T, int D, int FEAT, int HPW>
int launch_h(const DecodeArgs& args, hipStream_t stream) {
  constexpr bool F8 = (FEAT & kFp8) != 0;
  const int64_t items = (int64_t)(args.Hkv / HPW) * args.CG * args.B * args.S;
  const size_t lds = decode_lds_bytes<D, HPW, F8>(args.G);
  if (lds > 65536) {
    // (the fp8 D = 256 variants with two tiles per step use more than 64 KB);
    // raised once per device (the attribute is per device; concurrent first
    // calls may both set it, which is harmless)
    static std::atomic<uint64_t> attr_set{0};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return -3;
    if (!(attr_set.load() >> dev & 1)) {
      if (hipFuncSetAttribute(reinterpret_cast<const void*>(&decode_kernel<T, D, FEAT, HPW>),
                              hipFuncAttributeMaxDynamicSharedMemorySize,
                              static_cast<int>(decode_lds_bytes<D, HPW, F8>(16))) != hipSuccess)
        return -3;
      attr_set.fetch_or(uint64_t(1) << dev);
    }
  }
  hipLaunchKernelGGL((decode_kernel<T, D, FEAT, HPW>), dim3(static_cast<unsigned>(items)),
                     dim3(kWaves * 64), lds, stream, args);
  return hipGetLastError() == hipSuccess ? 0 : -3;
}

template <typename T, int D, int FEAT>
int launch_d(const DecodeArgs& args, hipStream_t stream) {
  if constexpr (D <= 128) {
    if (args.Hkv % 2 == 0 && 2 * args.G <= 16) return launch_h<T, D, FEAT, 2>(args, stream);
  }
  return launch_h<T, D, FEAT, 1>(args, stream);
}

template <typename T, int D, int F8>
int launch_feat(const DecodeArgs& a, bool softcap, bool alibi, hipStream_t s) {
  if (softcap && alibi) return launch_d<T, D, F8 | kSoftcap | kAlibi>(a, s);
  if (softcap) return launch_d<T, D, F8 | kSoftcap>(a, s);
  if (alibi) return launch_d<T, D, F8 | kAlibi>(a, s);
  return launch_d<T, D, F8>(a, s);
}

template <typename T, int F8>
int launch_t(const DecodeArgs& a, int D, bool softcap, bool alibi, hipStream_t s) {
  switch (D) {
    case 64: return launch_feat<T, 64, F8>(a, softcap, alibi, s);
    case 128: return launch_feat<T, 128, F8>(a, softcap, alibi, s);
    default: return launch_feat<T, 256, F8>(a, softcap, alibi, s);
  }
}

}  // namespace

int launch_decode(const AttnParams& p, hipStream_t stream) {
  if (p.num_seqs == 0) return 0;
  DecodeArgs a;
  a.out = p.out;
  a.lse = p.lse;
  a.part_out = p.part_out;
  a.part_lse = p.part_lse;
  a.q = static_cast<const uint16_t*>(p.q);
  a.kc = static_cast<const uint16_t*>(p.key_cache);
  a.vc = static_cast<const uint16_t*>(p.value_cache);
  a.seq_lens = p.seq_lens;
  a.block_table = p.block_table;
  a.bt_stride = p.block_table_stride;
  a.B = p.num_seqs;
  a.Hq = p.num_heads;
  a.Hkv = p.num_kv_heads;
  a.G = p.num_heads / p.num_kv_heads;
  a.CG = (a.G + 15) / 16;
  a.bs = p.block_size;
  a.S = p.num_splits;
  {
    // fixed, block-aligned chunks sized from the batch bound max_seq_len
    const int64_t per = ((int64_t)p.max_seqlen_k + p.num_splits - 1) / p.num_splits;
    a.chunk = static_cast<int>((per + p.block_size - 1) / p.block_size * p.block_size);
  }
  a.bs_magic = static_cast<uint32_t>(((1ULL << 32) + p.block_size - 1) / p.block_size);
  const bool softcap = p.softcap > 0.f;
  a.scale_log2 = p.scale * kLog2e;
  a.cap_k2 = softcap ? 2.0f * kLog2e * p.scale / p.softcap : 0.f;
  a.cap_log2 = p.softcap * kLog2e;
  a.window_left = p.window_left;
  a.alibi = p.alibi_slopes;
  a.sinks = p.sinks;
  a.k_scale = p.k_scale;
  a.v_scale = p.v_scale;
  a.q_scale = p.q_scale;
  a.counters = p.num_splits > 1 ? p.split_counters : nullptr;
  a.trace = trace_buffer();
  const bool alibi = p.alibi_slopes != nullptr;
  if (p.kv_fp8 && p.q_scale != nullptr) {
    if (p.dtype == kBF16) return launch_t<BF16, kFp8 | kQ8>(a, p.head_size, softcap, alibi, stream);
    return launch_t<F16, kFp8 | kQ8>(a, p.head_size, softcap, alibi, stream);
  }
  if (p.kv_fp8) {
    if (p.dtype == kBF16) return launch_t<BF16, kFp8>(a, p.head_size, softcap, alibi, stream);
    return launch_t<F16, kFp8>(a, p.head_size, softcap, alibi, stream);
  }
  if (p.dtype == kBF16) return launch_t<BF16, 0>(a, p.head_size, softcap, alibi, stream);
  return launch_t<F16, 0>(a, p.head_size, softcap, alibi, stream);
}

}  // namespace pa
