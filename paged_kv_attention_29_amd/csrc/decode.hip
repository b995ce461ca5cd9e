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
// queries), so each K/V byte is read from HBM once for all G heads.  Keys
// are processed in tiles of 16 (one MFMA M-tile); block_size is a multiple
// of 16, so a tile never straddles two cache blocks.
//
//   S^T[16 keys x 16 heads] = K_tile[16 x D] . Q^T[D x 16]    (mfma 16x16x32)
//   O^T[D x 16 heads]      += V_tile^T[D x 16] . P^T[16 x 16] (mfma 16x16x16)
//
// K is loaded from HBM straight into the A-operand layout (16-byte pieces of
// a key row per lane).  V needs its key index inside each lane, so each wave
// writes its V tile to a private LDS slab row-major and reads it back with
// the LDS transpose read (one ds_read_b64_tr_b16 per PV MFMA).  The 4 waves of a workgroup take interleaved tiles of the
// split with their own online-softmax state (fp32, base-2 exponent) and are
// merged through LDS at the end.  The loads of the next tile are issued
// before the current tile is computed.
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
  int chunk;            // keys per split (block-aligned, from the batch bound)
  uint32_t bs_magic;    // ceil(2^32 / bs)
  float scale_log2;     // scale * log2(e)
  float scale_over_cap; // scale / softcap
  float cap_log2;       // softcap * log2(e)
  int window_left;      // -1 = none
  const float* alibi;   // nullable
};

enum { kSoftcap = 1, kAlibi = 2 };
constexpr float kTau = 8.0f;  // lazy-rescale threshold (log2 units)

// A work item covers HPW adjacent KV heads (2 when the head counts allow it
// and D <= 128): each key row of the item is then 2 * 256 contiguous bytes,
// which the memory system streams faster than 256-byte rows 2 KB apart.
// Their query heads are the first G * HPW columns of the MFMA tile.
// Keys per iteration: NT MFMA row tiles of 16, so that a wave keeps 16 KB of
// K/V in flight while it computes the previous step (one tile for two heads
// or D = 256).
template <int D, int HPW>
constexpr int kNT = (D <= 128 && HPW == 1) ? 2 : 1;

// LDS: per-wave V slabs of 16 * NT rows (pitch D + 16 elements: the 32-byte
// pad spreads the 16 rows a transpose read touches over all banks), reused
// after the key loop for the cross-wave combine: [wave][head j < G][m, l, O].
template <int D, int HPW>
constexpr int kVPitch = HPW * D + 16;
template <int D, int HPW>
constexpr size_t decode_lds_bytes(int G) {
  const size_t v = (size_t)kWaves * 16 * kNT<D, HPW> * kVPitch<D, HPW> * 2;
  const size_t c = (size_t)kWaves * G * HPW * (D + 2) * 4;
  return v > c ? v : c;
}

template <int D>
constexpr int kMinBlocks = D <= 128 ? 2 : 1;

template <typename T, int D, int FEAT, int HPW>
__global__ __launch_bounds__(kWaves * 64, kMinBlocks<D>) void decode_kernel(DecodeArgs a) {
  constexpr bool SOFTCAP = FEAT & kSoftcap;
  constexpr bool ALIBI = FEAT & kAlibi;
  constexpr int KK = D / 32;   // QK mfma steps along D
  constexpr int DC = D / 16;   // PV output chunks of 16 rows of D
  constexpr int NT = kNT<D, HPW>;
  constexpr int KPS = 16 * NT; // keys per step
  constexpr int P = kVPitch<D, HPW>;
  extern __shared__ __attribute__((aligned(16))) char smem[];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int r16 = lane & 15;   // key row of the K piece / head column of the tile
  const int c4 = lane >> 4;    // which quarter: keys 4*c4..4*c4+3 of S^T, D piece of K

  // Item order: split-major; within split p the (KV-head group, sequence)
  // pairs are rotated by p groups.  Workgroup i runs on XCD i % 8 and, within
  // it, on the shader engines in turn, so without the rotation all splits of
  // a sequence would land on the same XCDs and engines and long sequences
  // would load some of them more than others.
  const int HG = a.Hkv / HPW;
  const int per_split = HG * a.B;
  const int split = blockIdx.x / per_split;
  int j = blockIdx.x - split * per_split - static_cast<int>((int64_t)split * HG % per_split);
  if (j < 0) j += per_split;
  const int g0 = (j % HG) * HPW;  // first KV head of the item
  const int b = j / HG;

  const int L = a.seq_lens[b];
  const int pos = L - 1;
  // split p covers keys [p * chunk, (p + 1) * chunk) of the sequence; the
  // last split also takes any keys past S * chunk
  const int lo = static_cast<int>(min((int64_t)split * a.chunk, (int64_t)L));
  const int hi = split == a.S - 1 ? L : min(lo + a.chunk, L);
  const int lo_vis = a.window_left >= 0 ? max(lo, pos - a.window_left) : lo;
  const int s_begin = lo_vis / KPS;
  const int s_end = (hi + KPS - 1) / KPS;
  const bool split_out = a.S > 1;
  if (lo_vis >= hi) {
    // no visible key: zero output, -inf log-sum-exp
    for (int idx = threadIdx.x; idx < a.G * HPW * D; idx += kWaves * 64) {
      const int h = g0 * a.G + idx / D;
      const int d = idx % D;
      if (split_out) {
        a.part_out[(((int64_t)split * a.B + b) * a.Hq + h) * D + d] = 0.f;
        if (d == 0) a.part_lse[((int64_t)split * a.Hq + h) * a.B + b] = kNegInf;
      } else {
        static_cast<uint16_t*>(a.out)[((int64_t)b * a.Hq + h) * D + d] = T::from_float(0.f);
        if (d == 0 && a.lse != nullptr) a.lse[(int64_t)h * a.B + b] = kNegInf;
      }
    }
    return;
  }

  const int GC = a.G * HPW;          // used columns
  const int head = g0 * a.G + r16;  // query head of this lane's column
  const bool col_ok = r16 < GC;
  const int hsel = r16 / a.G;       // which of the item's KV heads the column reads
  float slope_log2 = 0.0f;
  if constexpr (ALIBI) slope_log2 = col_ok ? a.alibi[head] * kLog2e : 0.0f;

  // Q^T as the B operand: column r16, D elements kk*32 + c4*8 .. +8; with
  // two KV heads, operand h is zero outside head h's columns, so the two
  // products accumulate into one S^T tile
  v8s qf[HPW][KK];
  {
    const uint16_t* qrow = a.q + ((int64_t)b * a.Hq + head) * D + c4 * 8;
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
      const v8s z = {0, 0, 0, 0, 0, 0, 0, 0};
      const v8s qv = col_ok ? *reinterpret_cast<const v8s*>(qrow + kk * 32) : z;
#pragma unroll
      for (int h = 0; h < HPW; ++h) qf[h][kk] = hsel == h ? qv : z;
    }
  }

  const int32_t* btab = a.block_table + (int64_t)b * a.bt_stride;
  const int64_t row_stride = (int64_t)a.Hkv * D;  // elements between consecutive slots
  const uint16_t* kcg = a.kc + (int64_t)g0 * D + c4 * 8;
  const uint16_t* vcg = a.vc + (int64_t)g0 * D + c4 * 8;

  struct Frag {
    v8s k[HPW][NT][KK];
    v8s v[HPW][NT][KK];
  };
  // Block ids of a step's tiles.  Loads are branch-free (so the compiler can
  // count outstanding loads exactly): a tile starting at or past hi is
  // clamped to the split's last tile, loaded, and fully masked.  The clamped
  // tile starts before hi, so it lies inside the sequence's last used block
  // at worst (block_size is a multiple of 16) and its block-table entry is
  // valid.
  const int last_j0 = hi > 0 ? ((hi - 1) & ~15) : 0;
  auto tile_j0 = [&](int step, int nt) { return min(step * KPS + 16 * nt, last_j0); };
  auto fetch_ids = [&](int step, int (&ids)[NT]) {
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) ids[nt] = btab[div_magic(tile_j0(step, nt), a.bs_magic)];
  };
  auto load_step = [&](int step, const int (&ids)[NT], Frag& f) {
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      const int j0 = tile_j0(step, nt);
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
  };

  float m_run = kNegInf;  // reference max (log2 units) of column r16
  float l_run = 0.0f;     // this lane's share of the running sum
  v4f o[DC];
#pragma unroll
  for (int dc = 0; dc < DC; ++dc) o[dc] = v4f{0.f, 0.f, 0.f, 0.f};

  uint16_t* vs = reinterpret_cast<uint16_t*>(smem) + wave * KPS * P;

  auto compute_step = [&](int step, const Frag& f) {
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
        for (int kk = 0; kk < KK; ++kk) sc = T::mfma16x16x32(f.k[h][nt][kk], qf[h][kk], sc);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int key = j0 + 4 * c4 + e;
        float v;
        if constexpr (SOFTCAP) v = a.cap_log2 * tanh_f32(sc[e] * a.scale_over_cap);
        else v = sc[e] * a.scale_log2;
        if constexpr (ALIBI) v -= slope_log2 * static_cast<float>(pos - key);
        x[nt][e] = (key >= lo_vis && key < hi) ? v : kNegInf;
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
#pragma unroll
      for (int dc = 0; dc < DC; ++dc) o[dc] *= alpha;
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
      const bool row_ok = key >= lo_vis && key < hi;
      uint16_t* dst = vs + (16 * nt + r16) * P + c4 * 8;
#pragma unroll
      for (int h = 0; h < HPW; ++h)
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) {
          const v8s z = {0, 0, 0, 0, 0, 0, 0, 0};
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
        const v4s lo = lds_read_tr16(vb + dc * 16);
        const v4s hi = lds_read_tr16(vb + 16 * P + dc * 16);
        const v8s av = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
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
  };

  // ---- double buffer: the next step's loads are in flight while the
  //      current one is computed.  Block ids run one step further ahead and
  //      are issued before the K/V loads, so waiting for them never waits for
  //      K/V data (the vector-memory counter completes in issue order).
  Frag cur, nxt;
  int ids[NT];
  int step = s_begin + wave;
  if (step < s_end) {
    fetch_ids(step, ids);
    load_step(step, ids, cur);
    fetch_ids(min(step + kWaves, s_end - 1), ids);
  }
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): Q and the first step landed
  for (; step < s_end; step += kWaves) {
    if (step + kWaves < s_end) {
      int ids2[NT];
      fetch_ids(min(step + 2 * kWaves, s_end - 1), ids2);
      load_step(step + kWaves, ids, nxt);
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) ids[nt] = ids2[nt];
    }
    compute_step(step, cur);
    cur = nxt;
  }

  // ---- combine the waves: lane holds O^T[d = dc*16 + 4*c4 + e][head r16]
  float l_tot = l_run + shfl_xor(l_run, 16);
  l_tot += shfl_xor(l_tot, 32);
  __syncthreads();  // every wave is done with its V slab
  float* comb = reinterpret_cast<float*>(smem);  // [wave][GC][D + 2]: m, l, O[D]
  constexpr int CP = D + 2;
  if (col_ok) {
    float* row = comb + (wave * GC + r16) * CP;
    if (c4 == 0) {
      row[0] = m_run;
      row[1] = l_tot;
    }
#pragma unroll
    for (int dc = 0; dc < DC; ++dc)
#pragma unroll
      for (int e = 0; e < 4; ++e) row[2 + dc * 16 + 4 * c4 + e] = o[dc][e];
  }
  __syncthreads();
  for (int idx = threadIdx.x; idx < GC * D; idx += kWaves * 64) {
    const int j = idx / D;
    const int d = idx - j * D;
    float M = kNegInf;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) M = fmaxf(M, comb[(w * GC + j) * CP]);
    float num = 0.f, den = 0.f;
    if (M != kNegInf) {
#pragma unroll
      for (int w = 0; w < kWaves; ++w) {
        const float* row = comb + (w * GC + j) * CP;
        const float fw = fast_exp2(row[0] - M);
        den += fw * row[1];
        num += fw * row[2 + d];
      }
    }
    const float val = den > 0.f ? num / den : 0.f;
    const int h = g0 * a.G + j;
    const float lse = den > 0.f ? (M + __log2f(den)) * kLn2 : kNegInf;
    if (split_out) {
      a.part_out[(((int64_t)split * a.B + b) * a.Hq + h) * D + d] = val;
      if (d == 0) a.part_lse[((int64_t)split * a.Hq + h) * a.B + b] = lse;
    } else {
      static_cast<uint16_t*>(a.out)[((int64_t)b * a.Hq + h) * D + d] = T::from_float(val);
      if (d == 0 && a.lse != nullptr) a.lse[(int64_t)h * a.B + b] = lse;
    }
  }
}

template <typename T, int D, int FEAT, int HPW>
int launch_h(const DecodeArgs& args, hipStream_t stream) {
  const int64_t grid = (int64_t)(args.Hkv / HPW) * args.B * args.S;
  hipLaunchKernelGGL((decode_kernel<T, D, FEAT, HPW>), dim3(static_cast<unsigned>(grid)),
                     dim3(kWaves * 64), (decode_lds_bytes<D, HPW>(args.G)), stream, args);
  return hipGetLastError() == hipSuccess ? 0 : -3;
}

template <typename T, int D, int FEAT>
int launch_d(const DecodeArgs& args, hipStream_t stream) {
  if constexpr (D <= 128) {
    if (args.Hkv % 2 == 0 && 2 * args.G <= 16) return launch_h<T, D, FEAT, 2>(args, stream);
  }
  return launch_h<T, D, FEAT, 1>(args, stream);
}

template <typename T, int D>
int launch_feat(const DecodeArgs& a, bool softcap, bool alibi, hipStream_t s) {
  if (softcap && alibi) return launch_d<T, D, kSoftcap | kAlibi>(a, s);
  if (softcap) return launch_d<T, D, kSoftcap>(a, s);
  if (alibi) return launch_d<T, D, kAlibi>(a, s);
  return launch_d<T, D, 0>(a, s);
}

template <typename T>
int launch_t(const DecodeArgs& a, int D, bool softcap, bool alibi, hipStream_t s) {
  switch (D) {
    case 64: return launch_feat<T, 64>(a, softcap, alibi, s);
    case 128: return launch_feat<T, 128>(a, softcap, alibi, s);
    default: return launch_feat<T, 256>(a, softcap, alibi, s);
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
  a.scale_over_cap = softcap ? p.scale / p.softcap : 0.f;
  a.cap_log2 = p.softcap * kLog2e;
  a.window_left = p.window_left;
  a.alibi = p.alibi_slopes;
  const bool alibi = p.alibi_slopes != nullptr;
  if (p.dtype == kBF16) return launch_t<BF16>(a, p.head_size, softcap, alibi, stream);
  return launch_t<F16>(a, p.head_size, softcap, alibi, stream);
}

}  // namespace pa
