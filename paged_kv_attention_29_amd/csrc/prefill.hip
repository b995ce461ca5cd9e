// paged_attn_prefill: variable-length attention of new query tokens over
// the paged KV cache (vLLM flash_attn.py (e2f56c3), FlashAttentionImpl
// .forward, flash_attn_varlen_func with block_table / seqused_k).
//
// Work item = (kv head g, sequence b, query tile).  A query tile is NW waves
// x 32 MFMA rows, a row being one (token, query head) pair of the
// G = Hq / Hkv query heads that share KV head g, so one K/V tile staged in
// LDS serves all G heads.  Per 64-key tile each wave computes
//   S^T[64 keys x 32 rows] = K[64 x D] . Q^T[D x 32]         (mfma 32x32x16)
//   O^T[D x 32 rows]      += V^T[D x 64] . P^T[64 x 32]      (mfma 32x32x16)
// With the query row as the MFMA N index, every lane holds one query row in
// both products, so the online-softmax row statistics are per lane (one
// cross-lane step pairs lane l with l ^ 32), and the probabilities of S^T
// become the B operand of the PV product in registers, without moving.
//
// K/V tiles go from HBM straight into LDS (global_load_lds_dwordx4: each
// lane's 16 bytes land at the wave's LDS base + 16 * lane), through a ring of
// NST stages, so NST - 1 tiles are in flight while one is computed and no
// registers hold data in transit.  Each wave fetches 64 / NW consecutive key
// rows of a tile; they lie in one 16-key group, hence in one cache block, so
// a wave needs one block-table entry per tile, fetched a tile before its K/V.
// Rows are stored unpadded with the 16-byte pieces of row R permuted (for
// D = 128, piece c at slot c ^ (R & 15) for K and c ^ 4 (R & 3) for V; see
// swz_k / swz_v): the K operand reads (16 rows at one piece index per 16
// lanes) and the V transpose reads (ds_read_b64_tr_b16, 4 rows x 4 pieces
// per 32 lanes) each cover all 64 banks.  Rows at or past the sequence end
// are fetched as a copy of its last row (finite, masked), so block-table
// padding and poisoned tails are never touched.
//
// The grid is a compact list of the query tiles (at most one empty slot per
// sequence), found by a wave-parallel search over cu_seqlens_q.  A
// workgroup's key tiles run in three parts: tiles that may cut a row's
// visible range run the masked code; the tiles all its rows see run the
// unmasked code two per pass, so each tile's ring stage (and the LDS read
// offsets) are constants.  An fp8 cache with an fp8 query computes S^T on
// the fp8 MFMA (32x32x64) straight from the staged codes; otherwise fp8
// tiles are widened to 16 bits in LDS first.
//
// Softmax work per score is kept to max, one fma, exp2, add and half a
// packed convert: the scale is folded into the exponent, masks are applied
// only on tiles that cut a row's visible range, tiles no row of a wave can
// see are skipped by that wave, and the running maximum is only moved (and
// the accumulators rescaled) when a row's maximum grows by more than 2^8
// (the result is exact either way: numerator and denominator share the
// same reference).
#include "common.h"
#include "launch.h"

#include <atomic>
#include <climits>      // INT_MAX, INT_MIN
#include <type_traits>  // std::true_type, std::integral_constant

namespace pa {

namespace {

constexpr int kKT = 64;       // keys per tile
constexpr float kTau = 8.0f;  // lazy-rescale threshold (log2 units)

enum { kSoftcap = 1, kAlibi = 2, kFp8 = 4, kQ8 = 8, kDual = 16 };
// instruction classes of __builtin_amdgcn_sched_group_barrier
constexpr int kSchedMfma = 0x008;
constexpr int kSchedDsRead = 0x100;

struct PrefillArgs {
  uint16_t* out;
  float* lse;
  const uint16_t* q;
  const uint16_t* kc;
  const uint16_t* vc;
  const int32_t* cu_q;
  const int32_t* seq_lens;
  const int32_t* block_table;
  int64_t bt_stride;
  int64_t total_q;
  // block-table columns readable from block_table (bt_stride, or fewer when
  // block_table points into the rows, past a shared prefix)
  int64_t bt_cols;
  // sequence c's queries are [cu_q[c], cu_q[c + cu_step]) (cu_step 1, or B
  // for the whole batch as one sequence) and its key count is
  // min(seq_lens[c] - len_sub, len_cap)
  int cu_step, len_sub, len_cap;
  int B, Hq, Hkv, G, bs, tok_per_tile;
  uint32_t bs_magic;
  float scale_log2;     // scale * log2(e)
  float cap_k2;         // 2 log2(e) scale / softcap
  float cap_log2;       // softcap * log2(e)
  int causal, window_left;
  const float* alibi;
  // key splits (grid z): split z takes keys [z * key_split, (z + 1) * key_split)
  // and writes its normalised partial result and LSE as part z of out / lse
  // ([splits, total_q, Hq, D] and [splits, Hq, total_q]); 0 = no split
  int key_split;
  // attention sinks [Hq] (fp32, nullable): one more logit per head in the
  // softmax denominator, without a value; folded into split 0 only
  const float* sinks;
  // fp8 (e4m3) cache: device fp32 scales (a stored code times the scale is
  // the K / V value); null for a 16-bit cache
  const float* k_scale;
  const float* v_scale;
  // fp8 query (with an fp8 cache): q holds e4m3 codes and this device fp32
  // scalar is their descale; null for a 16-bit query
  const float* q_scale;
  // timeline trace records (trace library only), or null
  uint64_t* trace;
  // workgroups along x of this problem's grid (key splits along z)
  int grid_x;
};

// A launch's arguments: one problem (p[0]), or, in the kDual variants, two
// independent problems in one grid: workgroups [0, n0) run p[0], the rest
// p[1], each numbered x fastest then z as in its own grid.  (The cascade
// runs its suffix and prefix passes this way, so that the short prefix
// workgroups fill the slots the suffix pass's uneven ones leave.)
struct PrefillLaunch {
  PrefillArgs p[2];
  int n0;
};

// Four waves (one per SIMD) per workgroup and a two-stage K/V ring, so
// several workgroups share a CU (two for D = 128, three for D = 64): one
// workgroup's Q loads and output stores overlap another's tiles.
template <int D>
constexpr int kNW = 4;  // waves per workgroup
template <int D>
constexpr int kNST = 2;  // LDS ring stages
template <int D>
constexpr int kMinWG = D == 64 ? 3 : D == 128 ? 2 : 1;  // workgroups per CU
template <int D>
constexpr int kRows = 32 * kNW<D>;     // MFMA rows per workgroup
template <int D>
constexpr int kTileBytes = kKT * D * 2;  // one of K or V
// An fp8 cache lands in the ring as codes (half the bytes per stage) and
// each tile is widened into one 16-bit K/V tile pair after the ring, which
// the MFMA operand reads use exactly as they use a 16-bit stage.
template <int D, bool F8>
constexpr size_t prefill_lds_bytes() {
  return F8 ? (size_t)kNST<D> * 2 * (kTileBytes<D> / 2) + 2 * kTileBytes<D>
            : (size_t)kNST<D> * 2 * kTileBytes<D>;
}

// LDS has 64 banks of 4 bytes: a ds_read_b128 serves 16 lanes per cycle and
// a ds_read_b64_tr_b16 32 lanes, and each such group must cover all 64
// banks.  A row of D = 128 fills the banks once; D = 64 rows pair up.
// K operand reads take 16 consecutive rows at one piece index: the 16 rows
// land on 16 distinct piece slots.
template <int D>
__device__ __forceinline__ int swz_k(int r) {
  return D == 64 ? (r >> 1) & 7 : r & 15;
}
// V transpose reads take 4 consecutive rows x 4 consecutive pieces per 32
// lanes: the 4 rows land on 4 distinct groups of 4 slots.  The swizzle only
// flips bits 2-3 of the piece index, so a piece's position is the lane's
// own offset plus an immediate.
template <int D>
__device__ __forceinline__ int swz_v(int r) {
  return D == 64 ? ((r >> 1) & 1) << 2 : (r & 3) << 2;
}

// fp8 K rows (D bytes) read as the fp8 MFMA's A operand: 16 consecutive
// rows at one 16-byte piece index per 16 lanes must cover all 64 banks,
// i.e. 256 / D rows share a bank line and the piece index is flipped by the
// row's line number within the 16.
template <int D>
__device__ __forceinline__ int swz8(int r) {
  return (r / (256 / D)) & (D / 16 - 1);
}
typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v4i __attribute__((ext_vector_type(4)));

// 16 bytes per lane from sbase + voff (global memory) into LDS at byte
// address lds_base + 16 * lane (global_load_lds_dwordx4; sbase and lds_base
// wave-uniform).  Issued as asm: a DMA the compiler knows of makes it wait
// for every LDS DMA in flight before each later LDS read, since it cannot
// tell the stages apart, which would empty the ring.  The DMA waits are
// placed by hand instead (wait_vmcnt before the hand-off barrier).  M0,
// which holds the LDS base, is restored afterwards.  The s_nop covers the
// GFX9 hazards of an LDS DMA that reads M0 right after an SALU write of M0
// (one wait state) and of a vector-memory instruction that reads an SGPR a
// VALU instruction wrote (five); without the first, the DMA can take the
// previous M0 as its LDS base.
__device__ __forceinline__ void dma16(const void* sbase, uint32_t voff, uint32_t lds_base) {
  // Both are wave-uniform; read from lane 0 so that the asm's scalar
  // operands are scalar registers whatever the register allocator did with
  // them (free when they already are).  readfirstlane works on int: each
  // half goes back through uint32_t, so the low half of the address is not
  // sign-extended into the high one.
  const uint64_t sb = reinterpret_cast<uint64_t>(sbase);
  const uint32_t lo = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<int>(sb)));
  const uint32_t hi = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<int>(sb >> 32)));
  sbase = reinterpret_cast<const void*>(static_cast<uint64_t>(hi) << 32 | lo);
  lds_base = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<int>(lds_base)));
  uint32_t save;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %1\n\t"
      "s_nop 4\n\t"
      "global_load_lds_dwordx4 %2, %3\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(save)
      : "s"(lds_base), "v"(voff), "s"(sbase));
}

// 16-byte global load the compiler does not track (no wait is inserted for
// its result): the caller waits with wait_vmcnt and then claims the value.
__device__ __forceinline__ v8s load16_async(const void* p) {
  v8s r;
  asm volatile("global_load_dwordx4 %0, %1, off" : "=v"(r) : "v"(p));
  return r;
}
// 8-byte global load the compiler does not track (same contract)
__device__ __forceinline__ u32x2 load8_async(const void* p) {
  u32x2 r;
  asm volatile("global_load_dwordx2 %0, %1, off" : "=v"(r) : "v"(p));
  return r;
}
// 4-byte global load the compiler does not track (same contract)
__device__ __forceinline__ uint32_t load4_async(const void* p) {
  uint32_t r;
  asm volatile("global_load_dword %0, %1, off" : "=v"(r) : "v"(p));
  return r;
}
// orders every use of r after the preceding (explicit) wait
__device__ __forceinline__ void claim(v8s& r) { asm volatile("" : "+v"(r)); }
__device__ __forceinline__ void claim(uint32_t& r) { asm volatile("" : "+v"(r)); }
__device__ __forceinline__ void claim(u32x2& r) { asm volatile("" : "+v"(r)); }

// max of v over lanes l and l ^ 32 (v_permlane32_swap exchanges the halves)
__device__ __forceinline__ float swap_halves_max(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

// Workgroup barrier for the LDS hand-off (a compiler memory barrier too).
// It drains this wave's LDS reads; the DMA waits come before it.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return static_cast<uint32_t>(
      reinterpret_cast<uintptr_t>((__attribute__((address_space(3))) const char*)(p)));
}

// Operand reads at an LDS byte address held as an integer: a lane's base
// address (in a register) plus a constant, which becomes the instruction's
// immediate offset.
using lds_v8s = __attribute__((address_space(3))) const v8s;
using lds_v4s = __attribute__((address_space(3))) v4s;
__device__ __forceinline__ v8s lds_load16(uint32_t addr) { return *(lds_v8s*)(addr); }
// ds_read_b64_tr_b16 (the lane layout of lds_read_tr16)
__device__ __forceinline__ v4s lds_load_tr16(uint32_t addr) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s*)(addr));
}

// wait until at most N vector-memory loads of this wave are outstanding
// (asm, so it stays ordered with the untracked loads and their claims)
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0)" ::"i"(N));
}

template <typename T, int D, int FEAT>
__global__ __launch_bounds__(kNW<D> * 64, kMinWG<D>) void prefill_kernel(PrefillLaunch launch) {
  constexpr bool DUAL = FEAT & kDual;
  // this workgroup's problem and its place in that problem's grid
  const int sel = DUAL && blockIdx.x >= static_cast<unsigned>(launch.n0) ? 1 : 0;
  PrefillArgs a = launch.p[sel];
  const unsigned lin = DUAL ? blockIdx.x - (sel ? launch.n0 : 0) : 0;
  const unsigned bx = DUAL ? lin % static_cast<unsigned>(a.grid_x) : blockIdx.x;
  const unsigned bz = DUAL ? lin / static_cast<unsigned>(a.grid_x) : blockIdx.z;
  constexpr bool SOFTCAP = FEAT & kSoftcap;
  constexpr bool ALIBI = FEAT & kAlibi;
  constexpr bool F8 = FEAT & kFp8;
  constexpr bool Q8 = FEAT & kQ8;  // fp8 query codes
  // fp8 query over an fp8 cache: S^T = K Q^T runs on the fp8 MFMA
  // (32x32x64, e4m3 x e4m3, exact products, fp32 sums) straight from the
  // staged fp8 K tile; only V is widened to 16 bits for the PV product
  constexpr bool QK8 = F8 && Q8;
  constexpr int K8S = D / 64;                // fp8 QK steps of 64 head dims
  constexpr int NQL = QK8 ? 2 * K8S : (D / 16);  // Q load instructions
  constexpr int NW = kNW<D>;
  constexpr int NST = kNST<D>;
  constexpr int TB = kTileBytes<D>;
  constexpr int KQ = D / 16;           // QK mfma steps along D
  constexpr int DC = D / 32;           // PV output chunks of 32 head dims
  constexpr int RB = 2 * D;            // bytes per key row of a 16-bit tile
  constexpr int RBC = F8 ? D : RB;     // bytes per key row as cached (and staged)
  constexpr int TBC = kKT * RBC;       // one of K or V as staged
  constexpr int RW = kKT / NW;         // key rows fetched per wave per tile
  constexpr int NI = RW * RBC / 1024;  // DMA instructions per wave per tile, each of K and V
  constexpr int ROWS_PER_I = 1024 / RBC;
  static_assert(NI >= 1 && RW <= 16, "tile split");
  extern __shared__ __attribute__((aligned(16))) char smem[];

  const uint64_t t_entry = kTrace ? trace_clock() : 0;
  const uint64_t r_entry = kTrace ? trace_realclock() : 0;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
  const int r32 = lane & 31;
  const int g2 = lane >> 5;
  float v_scale = 1.0f;
  if constexpr (F8) {
    // the K scale multiplies every score, the V scale the result
    const float ks = *a.k_scale;
    a.scale_log2 *= ks;
    a.cap_k2 *= ks;
    v_scale = *a.v_scale;
  }
  if constexpr (Q8) {
    // an fp8 query's descale multiplies every score too
    const float qs = *a.q_scale;
    a.scale_log2 *= qs;
    a.cap_k2 *= qs;
  }

  // Grid x = t * Hkv + g over a compact list of query tiles t: sequence b
  // owns tiles [S_b, S_b + n_b) with S_b = floor(cu_q[b] / tok) + b and
  // n_b = ceil(nq_b / tok), ranges that are disjoint, increase with b and
  // lie below floor(total_q / tok) + B, so the grid holds at most one empty
  // slot per sequence however uneven the lengths.  Workgroups are dispatched
  // to the 8 XCDs round-robin in linear order, so with 8 KV heads XCD g runs
  // every workgroup of head g; the sequence is the outer index, so an XCD
  // works through one sequence's query tiles together and the sequence's
  // K/V for that head stays in the XCD's L2 while they run.  Inside a
  // sequence the long (late) tiles go first.
  const int g = bx % a.Hkv;
  const int t = static_cast<int>(bx / a.Hkv);
  const int tok = a.tok_per_tile;
  // The last b with S_b <= t, by a wave-parallel search: each round splits
  // the candidate range [lo, lo + span) into 64 parts and keeps the last
  // part whose first S is <= t (one round up to 64 sequences, three up to
  // 2^18).  The final round also reads the sequence's bounds and length,
  // and the block id of this wave's first key group (keys RW * wave ..),
  // which the first tile needs whenever the key range starts at key 0.
  const int wave_blk = wave * RW / a.bs;  // block-table column of that group
  int lo = 0, span = a.B, q0 = 0, q1 = 0, L = 0, blk0 = 0;
  for (;;) {
    const int step = (span + 63) / 64;
    const int c = lo + lane * step;
    const bool in = lane * step < span;
    const bool fin = in && step == 1;
    const int cq = in ? a.cu_q[c] : 0;
    const int cq1 = fin ? a.cu_q[c + a.cu_step] : 0;
    const int cl = fin ? min(a.seq_lens[c] - a.len_sub, a.len_cap) : 0;
    const int cb = fin && wave_blk < a.bt_cols ? a.block_table[(int64_t)c * a.bt_stride + wave_blk] : 0;
    const int k = __builtin_popcountll(__builtin_amdgcn_ballot_w64(in && cq / tok + c <= t));
    if (k == 0) {  // below S_0 (cu_q[0] > 0)
      if (wave == 0) trace_put(a.trace, kTrEntry, t_entry);
      return;
    }
    lo += (k - 1) * step;
    if (step == 1) {
      q0 = __builtin_amdgcn_readlane(cq, k - 1);
      q1 = __builtin_amdgcn_readlane(cq1, k - 1);
      L = __builtin_amdgcn_readlane(cl, k - 1);
      blk0 = __builtin_amdgcn_readlane(cb, k - 1);
      break;
    }
    span = min(step, span - (k - 1) * step);
  }
  const int b = lo;
  const int nq = q1 - q0;
  const int local = t - (q0 / tok + b);
  if (local >= (nq + tok - 1) / tok) {  // an empty slot
    if constexpr (kTrace) {
      if (wave == 0) {
        trace_put(a.trace, kTrEntry, t_entry);
        trace_put(a.trace, kTrEnd, trace_clock());
        trace_hw(a.trace);
      }
    }
    return;
  }
  const int qt = (nq + tok - 1) / tok - 1 - local;
  const int tok0 = qt * tok;
  if constexpr (kTrace) {
    if (wave == 0) trace_put(a.trace, kTrItem, trace_clock());
  }
  const int ctx = L - nq;
  const int ntok = min(nq - tok0, a.tok_per_tile);
  const int p_first = ctx + tok0;
  const int p_last = p_first + ntok - 1;
  int k_hi = a.causal ? min(L, p_last + 1) : L;
  int k_lo = a.window_left >= 0 ? max(0, p_first - a.window_left) : 0;
  if (a.key_split > 0) {
    k_lo = max(k_lo, static_cast<int>(bz) * a.key_split);
    k_hi = min(k_hi, static_cast<int>(bz + 1) * a.key_split);
  }
  const int t_begin = k_lo / kKT;
  const int t_end = max((k_hi + kKT - 1) / kKT, t_begin);  // empty split: no tile

  // this lane's query row
  const int row = wave * 32 + r32;
  const int tk = row / a.G;
  const int hh = row - tk * a.G;
  const bool row_ok = tk < ntok;
  const int pos = ctx + tok0 + tk;
  const int head = g * a.G + hh;
  // positions of this wave's first and last valid rows (wave-uniform)
  const int w_tk0 = (wave * 32) / a.G;
  const int w_tk1 = min((wave * 32 + 31) / a.G, ntok - 1);
  const bool w_rows = w_tk0 < ntok;
  const int w_pmin = ctx + tok0 + w_tk0;
  const int w_pmax = ctx + tok0 + w_tk1;
  float slope_log2 = 0.0f;
  if constexpr (ALIBI) slope_log2 = row_ok ? a.alibi[head] * kLog2e : 0.0f;
  // keys visible to this row: lo_row <= key <= hi_row
  const int hi_row = a.causal ? min(pos, L - 1) : L - 1;
  const int lo_row = a.window_left >= 0 ? max(pos - a.window_left, 0) : 0;
  const uint32_t span_row = static_cast<uint32_t>(hi_row - lo_row);

  const int32_t* btab = a.block_table + (int64_t)b * a.bt_stride;
  // first key this wave fetches in a tile (clamped to the last key; the
  // other rows follow it inside the same 16-key group, hence the same block)
  auto group_key = [&](int tile) { return max(min(tile * kKT + wave * RW, L - 1), 0); };
  // Block ids of this wave's key group for tiles t0 + [0, 64): lane t holds
  // tile t0 + t (clamped to the last tile).  Loaded ahead in one vector load
  // and read with v_readlane, so the loop issues no scalar loads.
  auto load_ids = [&](int t0) -> uint32_t {
    const int tile = max(min(t0 + lane, t_end - 1), 0);
    return load4_async(btab + div_magic(group_key(tile), a.bs_magic));
  };
  const char* kc = reinterpret_cast<const char*>(a.kc) + (int64_t)g * RBC;
  const char* vc = reinterpret_cast<const char*>(a.vc) + (int64_t)g * RBC;

  // ---- DMA addressing.  Lane l of instruction i of this wave writes LDS
  //      bytes wave*RW*RB + i*1024 + 16*l of the tile: key row
  //      wave*RW + i*ROWS_PER_I + l/(RB/16), slot l % (RB/16).
  const uint32_t row_bytes = static_cast<uint32_t>(a.Hkv) * RBC;
  const uint32_t smem0 = lds_addr(smem);
  // the piece that belongs at this lane's slot of instruction i's row (an
  // fp8 stage is stored unpermuted, the widening pass applying the
  // swizzle, except an fp8 K stage that the fp8 MFMA reads itself)
  auto dma_row = [&](int i) { return wave * RW + i * ROWS_PER_I + lane / (RBC / 16); };
  auto dma_kp = [&](int i) {
    if constexpr (QK8) return ((lane % (RBC / 16)) ^ swz8<D>(dma_row(i))) * 16;
    return F8 ? (lane % (RBC / 16)) * 16 : ((lane % (RB / 16)) ^ swz_k<D>(dma_row(i))) * 16;
  };
  auto dma_vp = [&](int i) {
    return F8 ? (lane % (RBC / 16)) * 16 : ((lane % (RB / 16)) ^ swz_v<D>(dma_row(i))) * 16;
  };
  uint32_t dma_k[NI], dma_v[NI];  // byte offset from the wave's first row (all rows present)
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    const uint32_t rr = i * ROWS_PER_I + lane / (RBC / 16);
    dma_k[i] = rr * row_bytes + dma_kp(i);
    dma_v[i] = rr * row_bytes + dma_vp(i);
  }
  // block ids of this wave's key groups for 64 tiles (lane t: tile t0 + t)
  uint32_t ids = 0;
  // block id of relative tile jt (< 64 past the loaded chunk's start)
  auto id_of = [&](int jt) { return __builtin_amdgcn_readlane(static_cast<int>(ids), jt & 63); };
  auto issue_tile = [&](int tile, int blk, int stage) {
    const int kbase = tile * kKT;
    const int gk = group_key(tile);
    const int gq = div_magic(gk, a.bs_magic);
    const int64_t slot0 = (int64_t)blk * a.bs + (gk - gq * a.bs);  // cache slot of key gk
    const char* kb = kc + slot0 * row_bytes;
    const char* vb = vc + slot0 * row_bytes;
    const uint32_t kst = smem0 + stage * 2 * TBC + wave * RW * RBC;
    const uint32_t vst = kst + TBC;
    if (kbase + wave * RW + RW <= L) {
#pragma unroll
      for (int i = 0; i < NI; ++i) {
        dma16(kb, dma_k[i], kst + i * 1024);
        dma16(vb, dma_v[i], vst + i * 1024);
      }
    } else {
      // rows at or past the end repeat key L - 1
#pragma unroll
      for (int i = 0; i < NI; ++i) {
        const uint32_t rr = static_cast<uint32_t>(min(kbase + dma_row(i), L - 1) - gk);
        dma16(kb, rr * row_bytes + dma_kp(i), kst + i * 1024);
        dma16(vb, rr * row_bytes + dma_vp(i), vst + i * 1024);
      }
    }
  };

  // ---- prologue loads.  When the key range starts at key 0 and this wave's
  //      first group lies inside the sequence, tile 0's block id came with
  //      the sequence lookup and its K/V go out first; the block ids of the
  //      later tiles and Q follow.  Otherwise the ids come first and tile 0
  //      waits for them.  (t_begin < t_end whenever the tile has a query
  //      row, its own key being visible; only an empty key split has none.)
  static_assert(NST == 2, "the prologue fills one stage ahead");
  const int n = t_end - t_begin;
  const bool early = n > 0 && t_begin == 0 && wave * RW <= L - 1 && wave_blk < a.bt_cols;
  if (early) issue_tile(t_begin, blk0, 0);
  // (loaded unconditionally, an in-range entry even without tiles, so that
  // ids has one definition up to its claim after the prologue's wait: a
  // merge of two definitions could copy the register while it is loading)
  ids = load_ids(t_begin);
  // Q fragments (B operand of S^T = K Q^T).  Loaded by asm, like the K/V
  // DMA: a load the compiler tracks would get a wait at its first use that
  // also counts the DMAs in flight.  They complete before the prologue's
  // final wait (loads complete in order) and are claimed after it.
  v8s qf[KQ];
  u32x2 q8[Q8 && !QK8 ? KQ : 1];  // an fp8 query's codes, widened after the wait
  v8s q8x[QK8 ? 2 * K8S : 1];     // fp8 MFMA: its codes as B operands (2 x 16 bytes per step)
  {
    const int64_t qtok = row_ok ? q0 + tok0 + tk : q0;  // rows past the tile read a valid row
    if constexpr (QK8) {
      // step s: head dims 64 s + 32 g2 + [0, 32)
      const uint8_t* qrow =
          reinterpret_cast<const uint8_t*>(a.q) + (qtok * a.Hq + head) * D + 32 * g2;
#pragma unroll
      for (int i = 0; i < 2 * K8S; ++i) q8x[i] = load16_async(qrow + 64 * (i >> 1) + 16 * (i & 1));
    } else if constexpr (Q8) {
      const uint8_t* qrow =
          reinterpret_cast<const uint8_t*>(a.q) + (qtok * a.Hq + head) * D + 8 * g2;
#pragma unroll
      for (int kk = 0; kk < KQ; ++kk) q8[kk] = load8_async(qrow + 16 * kk);
    } else {
      const uint16_t* qrow = a.q + (qtok * a.Hq + head) * D + 8 * g2;
#pragma unroll
      for (int kk = 0; kk < KQ; ++kk) qf[kk] = load16_async(qrow + 16 * kk);
    }
  }
  if (!early && n > 0) {
    // tile 0's block id once the ids (issued before Q) landed: the wait and
    // the read are one asm block, so nothing reads the loading register
    int blk;
    asm volatile("s_waitcnt vmcnt(%1)\n\tv_readfirstlane_b32 %0, %2" : "=s"(blk) : "i"(NQL), "v"(ids));
    issue_tile(t_begin, blk, 0);
  }

  float m_run = kNegInf;   // reference maximum of the row (log2 units)
  float l_run = 0.0f;      // this lane's half of the row sum
  v16f oacc[DC];
#pragma unroll
  for (int dc = 0; dc < DC; ++dc)
#pragma unroll
    for (int e = 0; e < 16; ++e) oacc[dc][e] = 0.0f;

  // logits z: raw score (no softcap / ALiBi) scaled by cz in the exponent, or
  // the finished log2-unit logit with cz = 1
  const float cz = (SOFTCAP || ALIBI) ? 1.0f : a.scale_log2;
  // does any row of this wave see a key of the tile starting at kbase?
  // (wave-uniform: the bounds are kept in scalar registers)
  const int act_hi = __builtin_amdgcn_readfirstlane(!w_rows ? -1 : a.causal ? w_pmax : INT_MAX);
  const int act_lo = __builtin_amdgcn_readfirstlane(
      a.window_left >= 0 ? static_cast<int>(max(static_cast<int64_t>(w_pmin) - a.window_left - (kKT - 1),
                                                static_cast<int64_t>(INT_MIN)))
                         : INT_MIN);
  auto tile_active = [&](int kbase) { return kbase <= act_hi && kbase >= act_lo; };

  // ---- K operand of S^T = K Q^T: rows h2*32 + r32 of the tile, 16-byte piece
  //      2*kk + g2 (swizzled); rows r32 and 32 + r32 share the swizzle
  uint32_t k_lane[KQ];
#pragma unroll
  for (int kk = 0; kk < KQ; ++kk)
    k_lane[kk] = smem0 + r32 * RB + 16 * ((2 * kk + g2) ^ swz_k<D>(r32));
  // ---- the fp8 MFMA's K operand: rows h2*32 + r32 of the fp8 stage, head
  //      dims 64 s + 32 g2 + [0, 32) = 16-byte pieces 4 s + 2 g2 + t
  uint32_t k8_lane[QK8 ? 2 * K8S : 1];
  if constexpr (QK8) {
#pragma unroll
    for (int i = 0; i < 2 * K8S; ++i)
      k8_lane[i] = smem0 + r32 * RBC + 16 * ((4 * (i >> 1) + 2 * g2 + (i & 1)) ^ swz8<D>(r32));
  }

  // ---- V operand of O^T += V^T P^T: step s holds V[16s + 4*g2 + [0,4)][d] and
  //      V[16s + 8 + 4*g2 + [0,4)][d] for d = dc*32 + r32, two transpose reads.
  //      Lane j of each 16-lane group points at row k0 + j/4, head dims
  //      c0 + 4*(j%4) with c0 = dc*32 + 16*((lane >> 4) & 1).  With the
  //      swizzle, the 16-byte piece of head dim d = dc*32 + vd in row r is
  //      4*(dc ^ x) + vd/8 with x = swz_v(r)/4 < 4, i.e. lane address m = dc & 3
  //      plus the immediate 64*(dc & ~3).
  constexpr int NM = DC < 4 ? DC : 4;
  uint32_t v_lane[NM];
  {
    const int vr = 4 * g2 + ((lane & 15) >> 2);              // row within a 16-key step
    const int vd = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);  // head dim within a chunk
    const int x = swz_v<D>(vr) >> 2;
#pragma unroll
    for (int m = 0; m < NM; ++m)
      v_lane[m] = smem0 + vr * RB + 64 * (m ^ x) + 16 * (vd >> 3) + 2 * (vd & 7);
  }

  // ---- softmax of one tile's scores (lane holds keys
  //      kbase + 32*h2 + 8*(e/4) + 4*g2 + e%4 of its row): logits, masks
  //      (MASKED: the tile cuts a row's visible range), lazy rescale,
  //      probabilities packed as the B operand of the PV product
  float neg_m = 0.0f;  // -m_run, or 0 while m_run = -inf
  auto softmax = [&](v16f* sacc, int kbase, v8s* pb, auto masked_c) {
    constexpr bool MASKED = decltype(masked_c)::value;
#pragma unroll
    for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        float z = sacc[h2][e];
        const int key = kbase + 32 * h2 + 8 * (e >> 2) + 4 * g2 + (e & 3);
        if constexpr (SOFTCAP) z = softcap_log2(z, a.cap_k2, a.cap_log2);
        else if constexpr (ALIBI) z = z * a.scale_log2;
        if constexpr (ALIBI) z -= slope_log2 * static_cast<float>(abs(pos - key));
        sacc[h2][e] = z;
      }
    if constexpr (MASKED) {
      if (a.window_left < 0) {
        // one bound (no window): the key at offset o of the lane's pattern is
        // visible iff o <= hi_row - kbase - 4*g2 (o is an inline constant)
        const int lim = hi_row - kbase - 4 * g2;
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
          for (int e = 0; e < 16; ++e)
            sacc[h2][e] = 32 * h2 + 8 * (e >> 2) + (e & 3) <= lim ? sacc[h2][e] : kNegInf;
      } else {
        // visible iff 0 <= key - lo_row <= span_row (unsigned compare)
        const int base = kbase + 4 * g2 - lo_row;
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
          for (int e = 0; e < 16; ++e) {
            const uint32_t rel = static_cast<uint32_t>(base + 32 * h2 + 8 * (e >> 2) + (e & 3));
            sacc[h2][e] = rel <= span_row ? sacc[h2][e] : kNegInf;
          }
      }
    }
    // row max: three-input maxima over the lane's 32 scores (16 of them),
    // then the other half of the row (lane ^ 32) through a lane swap
    auto sc = [&](int i) { return sacc[i >> 4][i & 15]; };
    float m1[10];
#pragma unroll
    for (int i = 0; i < 10; ++i) m1[i] = fmaxf(fmaxf(sc(3 * i), sc(3 * i + 1)), sc(3 * i + 2));
    const float m2a = fmaxf(fmaxf(m1[0], m1[1]), m1[2]);
    const float m2b = fmaxf(fmaxf(m1[3], m1[4]), m1[5]);
    const float m2c = fmaxf(fmaxf(m1[6], m1[7]), m1[8]);
    const float m2d = fmaxf(fmaxf(m1[9], sc(30)), sc(31));
    const float mx = swap_halves_max(fmaxf(fmaxf(fmaxf(m2a, m2b), m2c), m2d));
    const float m_tile = mx * cz;

    // lazy rescale: move the reference only when the max grew a lot; rows
    // that do not grow keep alpha = 1
    const bool grow = m_tile > m_run + kTau;
    if (wave_any(grow)) {
      const float m_new = grow ? m_tile : m_run;
      const float alpha = grow ? fast_exp2(m_run - m_new) : 1.0f;  // 0 when m_run = -inf
      l_run *= alpha;
      // a row whose reference is still -inf has seen no key and holds zeros:
      // the accumulators need no scaling when every growing row is such a row
      // (the first tile of a wave)
      if (wave_any(grow && m_run != kNegInf)) {
#pragma unroll
        for (int dc = 0; dc < DC; ++dc) oacc[dc] *= alpha;
      }
      m_run = m_new;
      neg_m = m_run == kNegInf ? 0.0f : -m_run;
    }

    // probabilities; the row sum adds the rounded values the PV product
    // uses, in two chains (the first continues the running sum)
    float ps[2] = {l_run, 0.0f};
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      float pv[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) pv[e] = fast_exp2(fmaf(sacc[s >> 1][8 * (s & 1) + e], cz, neg_m));
      u32x4 w = {T::pack2(pv[0], pv[1]), T::pack2(pv[2], pv[3]), T::pack2(pv[4], pv[5]),
                 T::pack2(pv[6], pv[7])};
#pragma unroll
      for (int i = 0; i < 4; ++i) ps[s & 1] = T::sum2(w[i], ps[s & 1]);
      pb[s] = __builtin_bit_cast(v8s, w);
    }
    l_run = ps[0] + ps[1];
  };

  // The MFMA sections.  KOFF is the byte offset in LDS of the K tile the
  // operands are read from (the V tile follows it); where it is a constant
  // the per-lane addresses above take it as the reads' immediate offset.  Each
  // section is a scheduling region of its own (its read/MFMA interleave is
  // pinned) and runs at raised wave priority, so that while one wave of a
  // SIMD works through its MFMAs the other wave's softmax arithmetic fills
  // the issue slots between them.
  auto qk = [&](int KOFF, v16f* sacc) {
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
      for (int e = 0; e < 16; ++e) sacc[h2][e] = 0.0f;
    if constexpr (QK8) {
      // KOFF: the fp8 stage; per step and row half, 32 bytes of K codes
      v8s kf[4 * K8S];
#pragma unroll
      for (int i = 0; i < 2 * K8S; ++i)
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2) kf[2 * i + h2] = lds_load16(k8_lane[i] + KOFF + h2 * 32 * RBC);
#pragma unroll
      for (int st = 0; st < K8S; ++st)
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2) {
          const v8s lo = kf[2 * (2 * st) + h2], hi = kf[2 * (2 * st + 1) + h2];
          const v8i av = __builtin_shufflevector(__builtin_bit_cast(v4i, lo), __builtin_bit_cast(v4i, hi),
                                                 0, 1, 2, 3, 4, 5, 6, 7);
          const v8i bv = __builtin_shufflevector(__builtin_bit_cast(v4i, q8x[2 * st]),
                                                 __builtin_bit_cast(v4i, q8x[2 * st + 1]), 0, 1, 2, 3,
                                                 4, 5, 6, 7);
          // e4m3 x e4m3 (format 0 for both), unit scales (E8M0 127)
          sacc[h2] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(av, bv, sacc[h2], 0, 0, 0, 127,
                                                                     0, 127);
        }
      // schedule: 4 reads ahead, then one MFMA per two reads
      constexpr int NR = 4 * K8S, LEAD = 4, MID = (NR - LEAD) / 2;
      __builtin_amdgcn_sched_group_barrier(kSchedDsRead, LEAD, 0);
#pragma unroll
      for (int i = 0; i < MID; ++i) {
        __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 0);
        __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 2, 0);
      }
      __builtin_amdgcn_sched_group_barrier(kSchedMfma, 2 * K8S - MID, 0);
      __builtin_amdgcn_s_setprio(0);
      __builtin_amdgcn_sched_barrier(0);
      return;
    }
    // (reads written out first: the pinned interleave below then applies)
    v8s kf[2 * KQ];
#pragma unroll
    for (int kk = 0; kk < KQ; ++kk)
#pragma unroll
      for (int h2 = 0; h2 < 2; ++h2)
        kf[2 * kk + h2] = lds_load16(k_lane[kk] + KOFF + h2 * 32 * RB);
#pragma unroll
    for (int kk = 0; kk < KQ; ++kk)
#pragma unroll
      for (int h2 = 0; h2 < 2; ++h2) sacc[h2] = T::mfma32x32x16(kf[2 * kk + h2], qf[kk], sacc[h2]);
    // schedule: 6 reads ahead, then one MFMA per read
    constexpr int NR = 2 * KQ, LEAD = 6;
    __builtin_amdgcn_sched_group_barrier(kSchedDsRead, LEAD, 0);
#pragma unroll
    for (int i = 0; i < NR - LEAD; ++i) {
      __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 0);
      __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 1, 0);
    }
    __builtin_amdgcn_sched_group_barrier(kSchedMfma, LEAD, 0);
    __builtin_amdgcn_s_setprio(0);
    __builtin_amdgcn_sched_barrier(0);
  };
  auto pv = [&](int KOFF, const v8s* pb) {
    const int VOFF = KOFF + TB;
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int s = 0; s < 4; ++s)
#pragma unroll
      for (int dc = 0; dc < DC; ++dc) {
        const uint32_t p = v_lane[dc & 3] + VOFF + 16 * s * RB + 64 * (dc & ~3);
        const v4s lo = lds_load_tr16(p);
        const v4s hi = lds_load_tr16(p + 8 * RB);
        const v8s av = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        oacc[dc] = T::mfma32x32x16(av, pb[s], oacc[dc]);
      }
    // schedule: 8 reads ahead, then one MFMA per two reads
    constexpr int NR = 8 * DC, LEAD = 8, MID = (NR - LEAD) / 2;
    __builtin_amdgcn_sched_group_barrier(kSchedDsRead, LEAD, 0);
#pragma unroll
    for (int i = 0; i < MID; ++i) {
      __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 0);
      __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 2, 0);
    }
    __builtin_amdgcn_sched_group_barrier(kSchedMfma, 4 * DC - MID, 0);
    __builtin_amdgcn_s_setprio(0);
    __builtin_amdgcn_sched_barrier(0);
  };

  // ---- fp8 cache: widen this wave's RW rows of the staged K and V tiles
  //      (codes, unpermuted) into the 16-bit tile pair after the ring, with
  //      the operand swizzles, then a barrier.  Every wave widens its rows of
  //      every tile, also of tiles it skips itself.
  auto widen = [&](int stage) {
    // (with the fp8 MFMA only V is widened)
    const char* k8 = smem + stage * 2 * TBC;
    const char* v8 = k8 + TBC;
    char* k16 = smem + NST * 2 * TBC;
    char* v16 = k16 + TB;
    constexpr int PPR = D / 8;           // 8-element pieces per row
    constexpr int PPL = RW * PPR / 64;   // pieces per lane
    static_assert(PPL * 64 == RW * PPR, "widening split");
#pragma unroll
    for (int i = 0; i < PPL; ++i) {
      const int q = lane + 64 * i;
      const int r = wave * RW + q / PPR;
      const int c = q % PPR;
      if constexpr (!QK8) {
        const u32x2 kw = *reinterpret_cast<const u32x2*>(k8 + r * RBC + 8 * c);
        const v4s k0 = T::from_fp8x4(kw[0]), k1 = T::from_fp8x4(kw[1]);
        *reinterpret_cast<v8s*>(k16 + r * RB + 16 * (c ^ swz_k<D>(r))) =
            v8s{k0[0], k0[1], k0[2], k0[3], k1[0], k1[1], k1[2], k1[3]};
      }
      const u32x2 vw = *reinterpret_cast<const u32x2*>(v8 + r * RBC + 8 * c);
      const v4s v0 = T::from_fp8x4(vw[0]), v1 = T::from_fp8x4(vw[1]);
      *reinterpret_cast<v8s*>(v16 + r * RB + 16 * (c ^ swz_v<D>(r))) =
          v8s{v0[0], v0[1], v0[2], v0[3], v1[0], v1[1], v1[2], v1[3]};
    }
    lds_barrier();
  };

  // ---- the first tile, the block ids and Q landed
  wait_vmcnt<0>();
  claim(ids);
  lds_barrier();
  if constexpr (kTrace) {
    if (wave == 0) {
      trace_put(a.trace, kTrEntry, t_entry);
      trace_put(a.trace, kTrRealEntry, r_entry);
      trace_put(a.trace, kTrLoop0, trace_clock());
      trace_put(a.trace, kTrUnits, static_cast<uint64_t>(n));
      trace_put(a.trace, kTrWho, (uint64_t)b << 32 | static_cast<uint32_t>(qt));
      trace_hw(a.trace);
    }
  }
  if constexpr (QK8) {
#pragma unroll
    for (int i = 0; i < 2 * K8S; ++i) {
      claim(q8x[i]);
      const v8s z = {0, 0, 0, 0, 0, 0, 0, 0};  // (code 0 is +0)
      if (!row_ok) q8x[i] = z;
    }
  }
#pragma unroll
  for (int kk = 0; kk < (QK8 ? 0 : KQ); ++kk) {
    if constexpr (Q8 && !QK8) {
      claim(q8[kk]);
      const v4s lo = T::from_fp8x4(q8[kk][0]), hi = T::from_fp8x4(q8[kk][1]);
      qf[kk] = v8s{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    } else {
      claim(qf[kk]);
    }
    const v8s z = {0, 0, 0, 0, 0, 0, 0, 0};
    if (!row_ok) qf[kk] = z;
  }

  // ---- main loop over key tiles j: tile j + 1 goes into the stage of tile
  //      j - 1 (all waves passed the barrier after reading it); S^T, softmax
  //      and PV of tile j; then tile j + 1 must have landed before the
  //      barrier.  Tile j sits in ring stage j % 2.
  //
  //      The tiles are taken in three runs: [0, u0) and [u1, n) may cut a
  //      row's visible range (the window start, the causal diagonal, the
  //      sequence end) and run the masked tile code, skipping tiles no row
  //      of the wave sees; [u0, u1) is visible to every row of the
  //      workgroup and runs the unmasked code, two tiles per pass, so that
  //      each tile's stage is a constant.  A wave without query rows (the
  //      last tile of a sequence) only moves tiles through the ring.
  static_assert(NST == 2, "the loop alternates two ring stages");
  auto step = [&](int j, int stage, auto compute_c, auto masked_c) {
    const int tile = t_begin + j;
    const int kbase = tile * kKT;
    if (j + 1 < n) {
      const int jt = j + 1;
      if ((jt & 63) == 0) {  // next chunk of block ids (every 64 tiles)
        ids = load_ids(t_begin + jt);
        wait_vmcnt<0>();
        claim(ids);
      }
      issue_tile(tile + 1, id_of(jt), 1 - stage);
    }
    // LDS offset of the K tile the operand reads use (an fp8 stage is first
    // widened into the tile pair after the ring)
    const int koff = F8 ? NST * 2 * TBC : stage * 2 * TB;
    if constexpr (F8) widen(stage);
    if constexpr (decltype(compute_c)::value) {
      if (!decltype(masked_c)::value || tile_active(kbase)) {
        v16f sacc[2];
        v8s pb[4];
        qk(QK8 ? stage * 2 * TBC : koff, sacc);
        softmax(sacc, kbase, pb, masked_c);
        pv(koff, pb);
      }
    }
    // tile j + 1 landed (nothing else is in flight)
    wait_vmcnt<0>();
    lds_barrier();
  };
  if (w_rows) {
    // unmasked run: every key of the tile is visible to every query row of
    // the workgroup (positions p_first .. p_last)
    int u0 = t_begin, u1 = min(t_end, L / kKT);
    if (a.causal) u1 = min(u1, (p_first + 1) / kKT);
    if (a.window_left >= 0) {
      const int64_t lo = static_cast<int64_t>(p_last) - a.window_left;
      if (lo > 0) u0 = static_cast<int>(max(static_cast<int64_t>(u0), (lo + kKT - 1) / kKT));
    }
    u0 = min(u0, t_end) - t_begin;
    u1 = max(u1 - t_begin, u0);
    for (int j = 0; j < u0; ++j) step(j, j & 1, std::true_type{}, std::true_type{});
    int j = u0;
    if (j < u1 && (j & 1)) step(j++, 1, std::true_type{}, std::false_type{});
    for (; j + 1 < u1; j += 2) {
      step(j, 0, std::true_type{}, std::false_type{});
      step(j + 1, 1, std::true_type{}, std::false_type{});
    }
    if (j < u1) step(j++, 0, std::true_type{}, std::false_type{});
    for (; j < n; ++j) step(j, j & 1, std::true_type{}, std::true_type{});
  } else {
    for (int j = 0; j < n; ++j) step(j, j & 1, std::false_type{}, std::false_type{});
  }

  if constexpr (kTrace) {
    if (wave == 0) trace_put(a.trace, kTrLoop1, trace_clock());
  }
  // ---- epilogue: lane holds O^T[d = dc*32 + 8*(e/4) + 4*g2 + e%4][row]
  float l_tot = l_run + shfl_xor(l_run, 32);
  float m_fin = m_run, o_scale = 1.0f;
  if (a.sinks != nullptr && bz == 0) {
    // the sink as one more state (max sk, sum 1, output 0)
    const float sk = a.sinks[head] * kLog2e;
    const float M = fmaxf(m_run, sk);
    if (M != kNegInf) {
      o_scale = m_run == kNegInf ? 0.0f : fast_exp2(m_run - M);
      l_tot = l_tot * o_scale + fast_exp2(sk - M);
      m_fin = M;
    }
  }
  const float inv = l_tot > 0.f ? o_scale * v_scale * __builtin_amdgcn_rcpf(l_tot) : 0.0f;
  const int64_t part = bz;  // key split (0 without splits)
  // The wave's 32 output rows go through LDS (the ring is idle: every wave
  // passed the loop's last barrier and no DMA is in flight) so that the
  // global stores write whole rows, 16 bytes per lane: stored straight from
  // the accumulator layout, each store instruction would touch 32 rows with
  // 16 bytes apiece.
  constexpr int OP = D + 8;  // LDS row pitch in elements (16-byte pad)
  static_assert((size_t)kNW<D> * 32 * OP * 2 <= prefill_lds_bytes<D, false>(), "epilogue staging");
  uint16_t* ost = reinterpret_cast<uint16_t*>(smem) + wave * 32 * OP;
#pragma unroll
  for (int dc = 0; dc < DC; ++dc)
#pragma unroll
    for (int e4 = 0; e4 < 4; ++e4) {
      const v16f& v = oacc[dc];
      const u32x2 w = {T::pack2(v[4 * e4] * inv, v[4 * e4 + 1] * inv),
                       T::pack2(v[4 * e4 + 2] * inv, v[4 * e4 + 3] * inv)};
      *reinterpret_cast<u32x2*>(ost + r32 * OP + dc * 32 + 8 * e4 + 4 * g2) = w;
    }
  wave_lds_sync();
  constexpr int LPR = D / 8;     // lanes per row (16 bytes each)
  constexpr int RPI = 64 / LPR;  // rows per store instruction
#pragma unroll
  for (int i = 0; i < 32 / RPI; ++i) {
    const int r = i * RPI + lane / LPR;  // row of the wave
    const int c = (lane % LPR) * 8;
    const v8s val = *reinterpret_cast<const v8s*>(ost + r * OP + c);
    const int rr = wave * 32 + r;
    const int tk_r = rr / a.G;
    if (tk_r < ntok) {
      const int64_t qr = q0 + tok0 + tk_r;
      *reinterpret_cast<v8s*>(a.out + ((part * a.total_q + qr) * a.Hq + g * a.G + (rr - tk_r * a.G)) * D + c) = val;
    }
  }
  if (a.lse != nullptr && g2 == 0 && row_ok) {
    const int64_t qrow = q0 + tok0 + tk;
    a.lse[(part * a.Hq + head) * a.total_q + qrow] =
        l_tot > 0.f ? (m_fin + __log2f(l_tot)) * kLn2 : kNegInf;
  }
  if constexpr (kTrace) {
    const uint64_t t_end = trace_clock();
    if (wave == 0) {
      trace_put(a.trace, kTrEnd, t_end);
      trace_put(a.trace, kTrRealEnd, trace_realclock());
    }
    trace_put(a.trace, kTrWaveEnd + wave, t_end);
  }
}

// One problem of a launch: its arguments, its longest query run (0 = no
// work) and its number of key splits.
struct Problem {
  PrefillArgs a;
  int max_seqlen_q;
  int n_ksplits;
};

// Launches prefill_kernel<T, D, FEAT> over n problems (1, or 2 with kDual).
// Returns 0, -3 on a HIP error, or 1 when two problems do not fit one grid
// (the caller then launches them one by one).
template <typename T, int D, int FEAT>
int launch_p(const Problem* pr, int n, hipStream_t stream) {
  // the LDS limit of this kernel, raised once per device (the attribute is
  // per device; concurrent first calls may both set it, which is harmless)
  static std::atomic<uint64_t> attr_set{0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return -3;
  if (!(attr_set.load() >> dev & 1)) {
    if (hipFuncSetAttribute(reinterpret_cast<const void*>(&prefill_kernel<T, D, FEAT>),
                            hipFuncAttributeMaxDynamicSharedMemorySize,
                            static_cast<int>(prefill_lds_bytes<D, (FEAT & kFp8) != 0>())) != hipSuccess)
      return -3;
    attr_set.fetch_or(uint64_t(1) << dev);
  }
  PrefillLaunch L{};
  uint64_t wgs[2] = {0, 0};
  int splits[2] = {1, 1};
  for (int i = 0; i < n; ++i) {
    if (pr[i].max_seqlen_q == 0) {
      if (n == 1) return 0;
      return 1;
    }
    PrefillArgs a = pr[i].a;
    a.tok_per_tile = kRows<D> / a.G;
    // the compact tile list: floor(total_q / tokens per tile) + B slots per
    // KV head (the API bounds Hkv * (total_q + B) below 2^31)
    const int64_t slots = a.total_q / a.tok_per_tile + a.B;
    a.grid_x = static_cast<int>(a.Hkv * slots);
    splits[i] = a.key_split > 0 ? pr[i].n_ksplits : 1;
    wgs[i] = static_cast<uint64_t>(a.grid_x) * splits[i];
    L.p[i] = a;
  }
  dim3 grid(static_cast<unsigned>(L.p[0].grid_x), 1, static_cast<unsigned>(splits[0]));
  if (n == 2) {
    if (wgs[0] + wgs[1] > (uint64_t(1) << 22)) return 1;
    L.n0 = static_cast<int>(wgs[0]);
    grid = dim3(static_cast<unsigned>(wgs[0] + wgs[1]), 1, 1);
  }
  hipLaunchKernelGGL((prefill_kernel<T, D, FEAT>), grid, dim3(kNW<D> * 64),
                     (prefill_lds_bytes<D, (FEAT & kFp8) != 0>()), stream, L);
  return hipGetLastError() == hipSuccess ? 0 : -3;
}

// The kernel variant for a call's features, handed to fn as Inst<T, D, FEAT>
// (X: extra feature bits; kDual variants exist without ALiBi only).
template <typename T_, int D_, int FEAT_>
struct Inst {
  using T = T_;
  static constexpr int D = D_;
  static constexpr int FEAT = FEAT_;
};

template <typename T, int D, int X, typename Fn>
int by_feat(bool softcap, bool alibi, Fn& fn) {
  if constexpr (X & kDual) {
    if (alibi) return -3;
  } else {
    if (softcap && alibi) return fn(Inst<T, D, X | kSoftcap | kAlibi>{});
    if (alibi) return fn(Inst<T, D, X | kAlibi>{});
  }
  if (softcap) return fn(Inst<T, D, X | kSoftcap>{});
  return fn(Inst<T, D, X>{});
}

template <typename T, int X, typename Fn>
int by_head_size(int D, bool softcap, bool alibi, Fn& fn) {
  switch (D) {
    case 64: return by_feat<T, 64, X>(softcap, alibi, fn);
    case 128: return by_feat<T, 128, X>(softcap, alibi, fn);
    default: return by_feat<T, 256, X>(softcap, alibi, fn);
  }
}

template <int X, typename Fn>
int by_variant(const AttnParams& p, Fn& fn) {
  const bool softcap = p.softcap > 0.f, alibi = p.alibi_slopes != nullptr;
  const bool bf16 = p.dtype == kBF16;
  if (p.kv_fp8 && p.q_scale != nullptr)
    return bf16 ? by_head_size<BF16, X | kFp8 | kQ8>(p.head_size, softcap, alibi, fn)
                : by_head_size<F16, X | kFp8 | kQ8>(p.head_size, softcap, alibi, fn);
  if (p.kv_fp8)
    return bf16 ? by_head_size<BF16, X | kFp8>(p.head_size, softcap, alibi, fn)
                : by_head_size<F16, X | kFp8>(p.head_size, softcap, alibi, fn);
  return bf16 ? by_head_size<BF16, X>(p.head_size, softcap, alibi, fn)
              : by_head_size<F16, X>(p.head_size, softcap, alibi, fn);
}

Problem make_problem(const AttnParams& p) {
  PrefillArgs a{};
  a.out = static_cast<uint16_t*>(p.out);
  a.lse = p.lse;
  a.q = static_cast<const uint16_t*>(p.q);
  a.kc = static_cast<const uint16_t*>(p.key_cache);
  a.vc = static_cast<const uint16_t*>(p.value_cache);
  a.cu_q = p.cu_seqlens_q;
  a.seq_lens = p.seq_lens;
  a.block_table = p.block_table;
  a.bt_stride = p.block_table_stride;
  a.total_q = p.total_q;
  a.bt_cols = p.bt_cols > 0 ? p.bt_cols : p.block_table_stride;
  a.cu_step = p.cu_step > 0 ? p.cu_step : 1;
  a.len_sub = p.len_sub;
  a.len_cap = p.len_cap > 0 ? p.len_cap : INT_MAX;
  a.B = p.num_seqs;
  a.Hq = p.num_heads;
  a.Hkv = p.num_kv_heads;
  a.G = p.num_heads / p.num_kv_heads;
  a.bs = p.block_size;
  a.bs_magic = static_cast<uint32_t>(((1ULL << 32) + p.block_size - 1) / p.block_size);
  a.tok_per_tile = 0;  // set from the head size at launch
  const bool softcap = p.softcap > 0.f;
  a.scale_log2 = p.scale * kLog2e;
  a.cap_k2 = softcap ? 2.0f * kLog2e * p.scale / p.softcap : 0.f;
  a.cap_log2 = p.softcap * kLog2e;
  a.causal = p.causal;
  a.window_left = p.window_left;
  a.alibi = p.alibi_slopes;
  a.key_split = p.key_split;
  a.sinks = p.sinks;
  a.k_scale = p.k_scale;
  a.v_scale = p.v_scale;
  a.q_scale = p.q_scale;
  a.trace = trace_buffer();
  const int ns = p.key_split > 0 ? (p.max_seqlen_k + p.key_split - 1) / p.key_split : 1;
  return Problem{a, p.max_seqlen_q, ns};
}

}  // namespace

int launch_prefill(const AttnParams& p, hipStream_t stream) {
  if (p.num_seqs == 0 || p.total_q == 0) return 0;
  const Problem pr = make_problem(p);
  auto fn = [&](auto inst) {
    using I = decltype(inst);
    return launch_p<typename I::T, I::D, I::FEAT>(&pr, 1, stream);
  };
  return by_variant<0>(p, fn);
}

int launch_prefill_pair(const AttnParams& p0, const AttnParams& p1, hipStream_t stream) {
  if (p0.num_seqs == 0 || p0.total_q == 0 || p1.num_seqs == 0 || p1.total_q == 0) return 1;
  if (p0.dtype != p1.dtype || p0.head_size != p1.head_size || p0.kv_fp8 != p1.kv_fp8 ||
      (p0.q_scale != nullptr) != (p1.q_scale != nullptr) || (p0.softcap > 0.f) != (p1.softcap > 0.f) ||
      p0.alibi_slopes != nullptr || p1.alibi_slopes != nullptr)
    return 1;
  const Problem pr[2] = {make_problem(p0), make_problem(p1)};
  auto fn = [&](auto inst) {
    using I = decltype(inst);
    return launch_p<typename I::T, I::D, I::FEAT>(pr, 2, stream);
  };
  return by_variant<kDual>(p0, fn);
}

}  // namespace pa
