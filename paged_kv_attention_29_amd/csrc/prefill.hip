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
// Rows are stored unpadded with the 16-byte pieces of row R permuted
// (piece c at slot c ^ (R & 7) for K, c ^ 2 (R & 3) for V): the K operand
// reads (16 bytes of 8 rows at a time) and the V transpose reads
// (ds_read_b64_tr_b16, 32 bytes of 4 rows per 16 lanes) each hit distinct
// banks.  Rows at or past the sequence end are fetched as a copy of its
// last row (finite, masked), so block-table padding and poisoned tails are
// never touched.
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

#include <type_traits>

namespace pa {

namespace {

constexpr int kKT = 64;       // keys per tile
constexpr float kTau = 8.0f;  // lazy-rescale threshold (log2 units)

enum { kSoftcap = 1, kAlibi = 2 };

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
  int B, Hq, Hkv, G, bs, tok_per_tile;
  uint32_t bs_magic;
  float scale_log2;     // scale * log2(e)
  float scale_over_cap; // scale / softcap
  float cap_log2;       // softcap * log2(e)
  int causal, window_left;
  const float* alibi;
};

template <int D>
constexpr int kNW = D <= 128 ? 8 : 4;  // waves per workgroup (2 per SIMD / 1 per SIMD)
template <int D>
constexpr int kNST = D <= 128 ? 3 : 2;  // LDS ring stages
template <int D>
constexpr int kRows = 32 * kNW<D>;     // MFMA rows per workgroup
template <int D>
constexpr int kTileBytes = kKT * D * 2;  // one of K or V
template <int D>
constexpr size_t prefill_lds_bytes() { return (size_t)kNST<D> * 2 * kTileBytes<D>; }

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

// 16 bytes per lane from global memory into LDS at lds_base + 16 * lane
__device__ __forceinline__ void dma16(const void* src, void* lds_base) {
  __builtin_amdgcn_global_load_lds(src, (__attribute__((address_space(3))) void*)lds_base, 16, 0,
                                   0);
}

// Workgroup barrier for LDS hand-off.  __syncthreads() would make the
// compiler wait for every LDS DMA in flight (vmcnt(0)), which empties the
// ring; the DMA waits are placed explicitly instead, and this barrier only
// drains this wave's LDS reads.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// ds_read_b64_tr_b16 (see lds_read_tr16) at byte address addr + OFF.  Issued
// as asm so the compiler does not wait for the LDS DMA in flight before it
// (it cannot tell that the DMA writes another stage); the result must be
// claimed with lgkm_claim after the matching lgkm_wait.
template <int OFF>
__device__ __forceinline__ v4s ds_tr16(uint32_t addr) {
  v4s r;
  asm volatile("ds_read_b64_tr_b16 %0, %1 offset:%2" : "=v"(r) : "v"(addr), "i"(OFF));
  return r;
}
template <int N>
__device__ __forceinline__ void lgkm_wait() {
  asm volatile("s_waitcnt lgkmcnt(%0)" ::"i"(N));
}
// ties a register to the preceding lgkm_wait, so no use of it moves above
__device__ __forceinline__ void lgkm_claim(v4s& r) { asm volatile("" : "+v"(r)); }

template <int I>
using IC = std::integral_constant<int, I>;
// f(IC<I>{}) for I = B .. E-1, unrolled at compile time
template <int B, int E, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (B < E) {
    f(IC<B>{});
    static_for<B + 1, E>(f);
  }
}

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return static_cast<uint32_t>(
      reinterpret_cast<uintptr_t>((__attribute__((address_space(3))) const char*)(p)));
}

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  // s_waitcnt with vmcnt = N, expcnt and lgkmcnt at their maxima
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

template <typename T, int D, int FEAT>
__global__ __launch_bounds__(kNW<D> * 64, 1) void prefill_kernel(PrefillArgs a) {
  constexpr bool SOFTCAP = FEAT & kSoftcap;
  constexpr bool ALIBI = FEAT & kAlibi;
  constexpr int NW = kNW<D>;
  constexpr int NST = kNST<D>;
  constexpr int PD = NST - 1;          // tiles in flight ahead of the computed one
  constexpr int KQ = D / 16;           // QK mfma steps along D
  constexpr int DC = D / 32;           // PV output chunks of 32 head dims
  constexpr int RB = 2 * D;            // bytes per key row
  constexpr int RW = kKT / NW;         // key rows fetched per wave per tile
  constexpr int NI = RW * RB / 1024;   // DMA instructions per wave per tile, each of K and V
  constexpr int ROWS_PER_I = 1024 / RB;
  static_assert(NI >= 1 && RW <= 16, "tile split");
  extern __shared__ __attribute__((aligned(16))) char smem[];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
  const int r32 = lane & 31;
  const int g2 = lane >> 5;

  const int g = blockIdx.x;
  const int b = blockIdx.y;
  const int qt = gridDim.z - 1 - blockIdx.z;  // long (late) tiles first
  const int q0 = a.cu_q[b];
  const int nq = a.cu_q[b + 1] - q0;
  const int tok0 = qt * a.tok_per_tile;
  if (tok0 >= nq) return;
  const int L = a.seq_lens[b];
  const int ctx = L - nq;
  const int ntok = min(nq - tok0, a.tok_per_tile);
  const int p_first = ctx + tok0;
  const int p_last = p_first + ntok - 1;
  const int k_hi = a.causal ? min(L, p_last + 1) : L;
  const int k_lo = a.window_left >= 0 ? max(0, p_first - a.window_left) : 0;
  const int t_begin = k_lo / kKT;
  const int t_end = (k_hi + kKT - 1) / kKT;

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

  v8s qf[KQ];
  {
    const uint16_t* qrow = a.q + ((int64_t)(q0 + tok0 + tk) * a.Hq + head) * D + 8 * g2;
#pragma unroll
    for (int kk = 0; kk < KQ; ++kk) {
      v8s z = {0, 0, 0, 0, 0, 0, 0, 0};
      qf[kk] = row_ok ? *reinterpret_cast<const v8s*>(qrow + 16 * kk) : z;
    }
  }

  const int32_t* btab = a.block_table + (int64_t)b * a.bt_stride;
  const uint16_t* kc = a.kc + (int64_t)g * D;
  const uint16_t* vc = a.vc + (int64_t)g * D;

  // ---- DMA addressing.  Lane l of instruction i of this wave writes LDS
  //      bytes wave*RW*RB + i*1024 + 16*l of the tile: key row
  //      wave*RW + i*ROWS_PER_I + l/(RB/16), slot l % (RB/16).
  const uint32_t row_bytes = static_cast<uint32_t>(a.Hkv) * D * 2;
  int dma_row[NI];                // row of the tile this lane fetches, per instruction
  uint32_t dma_k[NI], dma_v[NI];  // byte offset from the wave's first row (all rows present)
  uint32_t dma_kp[NI], dma_vp[NI];  // byte offset of the piece within its row
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    const int rr = i * ROWS_PER_I + lane / (RB / 16);
    const int r = wave * RW + rr;
    const int slot = lane % (RB / 16);
    dma_row[i] = r;
    dma_kp[i] = (slot ^ swz_k<D>(r)) * 16;  // the piece that belongs at this slot
    dma_vp[i] = (slot ^ swz_v<D>(r)) * 16;
    dma_k[i] = rr * row_bytes + dma_kp[i];
    dma_v[i] = rr * row_bytes + dma_vp[i];
  }
  // first key this wave fetches in a tile (clamped to the last key; the
  // other rows follow it inside the same 16-key group, hence the same block)
  auto group_key = [&](int tile) { return min(tile * kKT + wave * RW, L - 1); };
  // (a scalar load: the entry is wave-uniform and the table is read-only)
  auto fetch_id = [&](int tile) -> int {
    const int idx = div_magic(group_key(min(tile, t_end - 1)), a.bs_magic);
    return *(const __attribute__((address_space(4))) int32_t*)(btab + idx);
  };
  auto issue_tile = [&](int tile, int blk, int stage) {
    const int kbase = tile * kKT;
    const int gk = group_key(tile);
    const int gq = div_magic(gk, a.bs_magic);
    const int64_t slot0 = (int64_t)blk * a.bs + (gk - gq * a.bs);  // cache slot of key gk
    const char* kb = reinterpret_cast<const char*>(kc) + slot0 * row_bytes;
    const char* vb = reinterpret_cast<const char*>(vc) + slot0 * row_bytes;
    char* kst = smem + stage * 2 * kTileBytes<D> + wave * RW * RB;
    char* vst = kst + kTileBytes<D>;
    if (kbase + wave * RW + RW <= L) {
#pragma unroll
      for (int i = 0; i < NI; ++i) {
        dma16(kb + dma_k[i], kst + i * 1024);
        dma16(vb + dma_v[i], vst + i * 1024);
      }
    } else {
      // rows at or past the end repeat key L - 1
#pragma unroll
      for (int i = 0; i < NI; ++i) {
        const uint32_t rr = static_cast<uint32_t>(min(kbase + dma_row[i], L - 1) - gk);
        dma16(kb + (rr * row_bytes + dma_kp[i]), kst + i * 1024);
        dma16(vb + (rr * row_bytes + dma_vp[i]), vst + i * 1024);
      }
    }
  };

  float m_run = kNegInf;   // reference maximum of the row (log2 units)
  float l_run = 0.0f;      // this lane's half of the row sum
  v16f oacc[DC];
#pragma unroll
  for (int dc = 0; dc < DC; ++dc)
#pragma unroll
    for (int e = 0; e < 16; ++e) oacc[dc][e] = 0.0f;

  // ---- prologue: block ids of the first PD + 1 tiles, then the first PD tiles
  // (t_begin < t_end whenever the tile has a query row: its own key is visible)
  int ids[PD + 1];
#pragma unroll
  for (int p = 0; p <= PD; ++p) ids[p] = fetch_id(t_begin + p);
#pragma unroll
  for (int p = 0; p < PD; ++p)
    if (t_begin + p < t_end) issue_tile(t_begin + p, ids[p], p);
  // the first tile (and Q) landed; the other issued tiles may stay in flight
  static_assert(PD <= 2, "prologue wait assumes at most two tiles in flight");
  if (PD == 2 && t_begin + 1 < t_end) wait_vmcnt<(PD - 1) * 2 * NI>();
  else wait_vmcnt<0>();
  lds_barrier();

  // logits z: raw score (no softcap / ALiBi) scaled by cz in the exponent, or
  // the finished log2-unit logit with cz = 1
  const float cz = (SOFTCAP || ALIBI) ? 1.0f : a.scale_log2;
  // K operand rows r32 and 32 + r32 share the swizzle (they differ by 32)
  const int krow_sw = swz_k<D>(r32);

  int stage = 0;
  for (int tile = t_begin; tile < t_end; ++tile) {
    const bool more = tile + PD < t_end;
    if (more) {
      const int next_id = fetch_id(tile + PD + 1);
      issue_tile(tile + PD, ids[PD], (stage + PD) % NST);
#pragma unroll
      for (int p = 0; p < PD - 1; ++p) ids[p + 1] = ids[p + 2];
      ids[PD] = next_id;
    }

    const int kbase = tile * kKT;
    bool active = w_rows;
    if (a.causal) active = active && kbase <= w_pmax;
    if (a.window_left >= 0) active = active && kbase + kKT - 1 >= w_pmin - a.window_left;

    if (active) {
      const uint16_t* ks = reinterpret_cast<const uint16_t*>(smem + stage * 2 * kTileBytes<D>);
      const uint16_t* vs = ks + kTileBytes<D> / 2;

      // ---- S^T = K Q^T for keys kbase + [0, 32) and [32, 64)
      v16f sacc[2];
#pragma unroll
      for (int h2 = 0; h2 < 2; ++h2) {
#pragma unroll
        for (int e = 0; e < 16; ++e) sacc[h2][e] = 0.0f;
        const uint16_t* krow = ks + (h2 * 32 + r32) * D;
#pragma unroll
        for (int kk = 0; kk < KQ; ++kk)
          sacc[h2] = T::mfma32x32x16(
              *reinterpret_cast<const v8s*>(krow + (((2 * kk + g2) ^ krow_sw) << 3)), qf[kk],
              sacc[h2]);
      }

      // ---- logits; lane holds keys kbase + 32*h2 + 8*(e/4) + 4*g2 + e%4 of its row
      const bool need_mask = kbase + kKT > L || (a.causal && kbase + kKT - 1 > w_pmin) ||
                             (a.window_left >= 0 && kbase < w_pmax - a.window_left);
#pragma unroll
      for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          float z = sacc[h2][e];
          const int key = kbase + 32 * h2 + 8 * (e >> 2) + 4 * g2 + (e & 3);
          if constexpr (SOFTCAP) z = a.cap_log2 * tanh_f32(z * a.scale_over_cap);
          else if constexpr (ALIBI) z = z * a.scale_log2;
          if constexpr (ALIBI) z -= slope_log2 * static_cast<float>(abs(pos - key));
          sacc[h2][e] = z;
        }
      if (need_mask) {
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
      float mx = kNegInf;
#pragma unroll
      for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
        for (int e = 0; e < 16; ++e) mx = fmaxf(mx, sacc[h2][e]);
      mx = fmaxf(mx, shfl_xor(mx, 32));
      const float m_tile = mx * cz;

      // ---- lazy rescale: move the reference only when the max grew a lot;
      //      rows that do not grow keep alpha = 1
      const bool grow = m_tile > m_run + kTau;
      if (wave_any(grow)) {
        const float m_new = grow ? m_tile : m_run;
        const float alpha = grow ? fast_exp2(m_run - m_new) : 1.0f;  // 0 when m_run = -inf
        l_run *= alpha;
#pragma unroll
        for (int dc = 0; dc < DC; ++dc) oacc[dc] *= alpha;
        m_run = m_new;
      }
      const float neg_m = m_run == kNegInf ? 0.0f : -m_run;

      float psum = 0.0f;  // sum of the rounded probabilities the PV product uses
      v8s pb[4];
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        float pv[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) pv[e] = fast_exp2(fmaf(sacc[s >> 1][8 * (s & 1) + e], cz, neg_m));
        u32x4 w = {T::pack2(pv[0], pv[1]), T::pack2(pv[2], pv[3]), T::pack2(pv[4], pv[5]),
                   T::pack2(pv[6], pv[7])};
#pragma unroll
        for (int e = 0; e < 4; ++e) psum = T::sum2(w[e], psum);
        pb[s] = __builtin_bit_cast(v8s, w);
      }
      l_run += psum;

      // ---- O^T += V^T P^T; the A operand of step s holds V[16s + 4*g2 + [0,4)][d] and
      //      V[16s + 8 + 4*g2 + [0,4)][d] for d = dc*32 + r32: two transpose reads.
      //      Lane j of each 16-lane group points at row k0 + j/4, head dims
      //      c0 + 4*(j%4) with c0 = dc*32 + 16*((lane >> 4) & 1).  With the
      //      swizzle, the 16-byte piece of head dim d = dc*32 + vd in row r is
      //      4*(dc ^ x) + vd/8 with x = swz_v(r)/4 < 4, i.e. lane address m = dc & 3
      //      plus the immediate 64*(dc & ~3).
      {
        const int vr = 4 * g2 + ((lane & 15) >> 2);              // row within a 16-key step
        const int vd = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);  // head dim within a chunk
        const uint32_t vbase = lds_addr(vs) + vr * RB + 16 * (vd >> 3) + 2 * (vd & 7);
        const int x = swz_v<D>(vr) >> 2;
        constexpr int NM = DC < 4 ? DC : 4;
        uint32_t va[NM];
#pragma unroll
        for (int m = 0; m < NM; ++m) va[m] = vbase + 64 * (m ^ x);
        v4s buf[2][2 * DC];
        // the 2 * DC reads of step S into b
        auto issue = [&](auto s_c, v4s* bb) {
          constexpr int S = decltype(s_c)::value;
          static_for<0, DC>([&](auto dc_c) {
            constexpr int dc = decltype(dc_c)::value;
            constexpr int off = 16 * S * RB + 64 * (dc & ~3);
            bb[2 * dc] = ds_tr16<off>(va[dc & 3]);
            bb[2 * dc + 1] = ds_tr16<off + 8 * RB>(va[dc & 3]);
          });
        };
        issue(IC<0>{}, buf[0]);
        static_for<0, 4>([&](auto s_c) {
          constexpr int S = decltype(s_c)::value;
          // reads of step S + 1 go out before step S's products
          if constexpr (S + 1 < 4) {
            issue(IC<S + 1>{}, buf[(S + 1) & 1]);
            lgkm_wait<(2 * DC < 15 ? 2 * DC : 15)>();  // (15: the field maximum)
          } else {
            lgkm_wait<0>();
          }
#pragma unroll
          for (int dc = 0; dc < DC; ++dc) {
            v4s& lo = buf[S & 1][2 * dc];
            v4s& hi = buf[S & 1][2 * dc + 1];
            lgkm_claim(lo);
            lgkm_claim(hi);
            const v8s av = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
            oacc[dc] = T::mfma32x32x16(av, pb[S], oacc[dc]);
          }
        });
      }
    }

    // the next tile landed (later ones may stay in flight); all waves are
    // done reading the stage the next DMA reuses
    if (more) wait_vmcnt<(PD - 1) * 2 * NI>();
    else wait_vmcnt<0>();
    lds_barrier();
    stage = stage + 1 == NST ? 0 : stage + 1;
  }

  // ---- epilogue: lane holds O^T[d = dc*32 + 8*(e/4) + 4*g2 + e%4][row]
  const float l_tot = l_run + shfl_xor(l_run, 32);
  if (!row_ok) return;
  const float inv = l_tot > 0.f ? __builtin_amdgcn_rcpf(l_tot) : 0.0f;
  const int64_t qrow = q0 + tok0 + tk;
  uint16_t* orow = a.out + (qrow * a.Hq + head) * D + 4 * g2;
#pragma unroll
  for (int dc = 0; dc < DC; ++dc)
#pragma unroll
    for (int e4 = 0; e4 < 4; ++e4) {
      const v16f& v = oacc[dc];
      u32x2 w = {T::pack2(v[4 * e4] * inv, v[4 * e4 + 1] * inv),
                 T::pack2(v[4 * e4 + 2] * inv, v[4 * e4 + 3] * inv)};
      *reinterpret_cast<u32x2*>(orow + dc * 32 + 8 * e4) = w;
    }
  if (a.lse != nullptr && g2 == 0)
    a.lse[(int64_t)head * a.total_q + qrow] =
        l_tot > 0.f ? (m_run + __log2f(l_tot)) * kLn2 : kNegInf;
}

template <typename T, int D, int FEAT>
int launch_p(const PrefillArgs& args, int max_seqlen_q, hipStream_t stream) {
  static bool attr_set = false;
  if (!attr_set) {
    attr_set = hipFuncSetAttribute(reinterpret_cast<const void*>(&prefill_kernel<T, D, FEAT>),
                                   hipFuncAttributeMaxDynamicSharedMemorySize,
                                   static_cast<int>(prefill_lds_bytes<D>())) == hipSuccess;
  }
  PrefillArgs a = args;
  a.tok_per_tile = kRows<D> / a.G;
  const int ntiles = (max_seqlen_q + a.tok_per_tile - 1) / a.tok_per_tile;
  if (ntiles == 0) return 0;
  const dim3 grid(a.Hkv, a.B, ntiles);
  hipLaunchKernelGGL((prefill_kernel<T, D, FEAT>), grid, dim3(kNW<D> * 64),
                     prefill_lds_bytes<D>(), stream, a);
  return hipGetLastError() == hipSuccess ? 0 : -3;
}

template <typename T, int D>
int launch_feat(const PrefillArgs& a, int mq, bool softcap, bool alibi, hipStream_t s) {
  if (softcap && alibi) return launch_p<T, D, kSoftcap | kAlibi>(a, mq, s);
  if (softcap) return launch_p<T, D, kSoftcap>(a, mq, s);
  if (alibi) return launch_p<T, D, kAlibi>(a, mq, s);
  return launch_p<T, D, 0>(a, mq, s);
}

template <typename T>
int launch_t(const PrefillArgs& a, int D, int mq, bool softcap, bool alibi, hipStream_t s) {
  switch (D) {
    case 64: return launch_feat<T, 64>(a, mq, softcap, alibi, s);
    case 128: return launch_feat<T, 128>(a, mq, softcap, alibi, s);
    default: return launch_feat<T, 256>(a, mq, softcap, alibi, s);
  }
}

}  // namespace

int launch_prefill(const AttnParams& p, hipStream_t stream) {
  if (p.num_seqs == 0 || p.total_q == 0) return 0;
  PrefillArgs a;
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
  a.B = p.num_seqs;
  a.Hq = p.num_heads;
  a.Hkv = p.num_kv_heads;
  a.G = p.num_heads / p.num_kv_heads;
  a.bs = p.block_size;
  a.bs_magic = static_cast<uint32_t>(((1ULL << 32) + p.block_size - 1) / p.block_size);
  a.tok_per_tile = 0;  // set from the head size at launch
  const bool softcap = p.softcap > 0.f;
  a.scale_log2 = p.scale * kLog2e;
  a.scale_over_cap = softcap ? p.scale / p.softcap : 0.f;
  a.cap_log2 = p.softcap * kLog2e;
  a.causal = p.causal;
  a.window_left = p.window_left;
  a.alibi = p.alibi_slopes;
  const bool alibi = p.alibi_slopes != nullptr;
  if (p.dtype == kBF16) return launch_t<BF16>(a, p.head_size, p.max_seqlen_q, softcap, alibi, stream);
  return launch_t<F16>(a, p.head_size, p.max_seqlen_q, softcap, alibi, stream);
}

}  // namespace pa
