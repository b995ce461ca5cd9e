// paged_attn_prefill: variable-length attention of new query tokens over
// the paged KV cache (vLLM flash_attn.py (e2f56c3), FlashAttentionImpl
// .forward, flash_attn_varlen_func with block_table / seqused_k).
//
// Work item = (kv head g, sequence b, query tile).  A query tile is 128 MFMA
// rows = (128 / G) tokens x the G query heads sharing KV head g, so one K/V
// tile staged in LDS serves all G heads.  Each of the 4 waves owns 32 rows
// and computes, per 64-key tile,
//   S^T[64 keys x 32 rows] = K[64 x D] . Q^T[D x 32]         (mfma 32x32x16)
//   O^T[D x 32 rows]      += V^T[D x 64] . P^T[64 x 32]      (mfma 32x32x16)
// With the query row as the MFMA N index, every lane holds one query row in
// both products, so the online-softmax row statistics are per lane (one
// cross-lane step pairs lane l with l ^ 32), and the probabilities of S^T
// become the B operand of the PV product in registers, without moving.
//
// Softmax work per score is kept to max, one fma, exp2, add and half a
// packed convert: the scale is folded into the exponent, masks are applied
// only on tiles that cut a row's visible range, tiles no row of a wave can
// see are skipped by that wave, and the running maximum is only moved (and
// the accumulators rescaled) when a row's maximum grows by more than 2^8
// (the result is exact either way: numerator and denominator share the
// same reference).
//
// K/V tiles are gathered block by block through the block table into
// registers one tile ahead (16 consecutive lanes per 16-byte pieces of a key
// row), then stored row-major to a double-buffered LDS stage.  The PV A
// operand needs V with the key index inside the lane; it is read with the
// LDS transpose read (ds_read_b64_tr_b16), two per MFMA.  Keys at or past the
// sequence end are never loaded (zero in LDS), so block-table padding and
// poisoned tails are never touched.
#include "common.h"
#include "launch.h"

namespace pa {

namespace {

constexpr int kPW = 4;      // waves per workgroup
constexpr int kRows = 128;  // MFMA rows per workgroup
constexpr int kKT = 64;     // keys per tile
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
constexpr int kKPitch = D + 8;      // K and V rows: 16-byte pad spreads rows over banks
template <int D>
constexpr int kStageBytes = 2 * kKT * kKPitch<D> * 2;
template <int D>
constexpr size_t prefill_lds_bytes() { return 2 * (size_t)kStageBytes<D>; }
template <int D>
constexpr int kMinBlocks = D <= 128 ? 2 : 1;

template <typename T, int D, int FEAT>
__global__ __launch_bounds__(kPW * 64, kMinBlocks<D>) void prefill_kernel(PrefillArgs a) {
  constexpr bool SOFTCAP = FEAT & kSoftcap;
  constexpr bool ALIBI = FEAT & kAlibi;
  constexpr int KQ = D / 16;        // QK mfma steps along D
  constexpr int DC = D / 32;        // PV output chunks of 32 head dims
  constexpr int V8 = D / 8;         // 16-byte pieces per row
  constexpr int V8_SHIFT = D == 64 ? 3 : (D == 128 ? 4 : 5);
  constexpr int LPT = kKT * V8 / (kPW * 64);  // pieces per thread per tile (K and V each)
  constexpr int KP = kKPitch<D>;
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
  const int64_t row_stride = (int64_t)a.Hkv * D;
  const uint16_t* kc = a.kc + (int64_t)g * D;
  const uint16_t* vc = a.vc + (int64_t)g * D;
  auto slot_of = [&](int j) -> int64_t {
    const int q = div_magic(j, a.bs_magic);
    return (int64_t)btab[q] * a.bs + (j - q * a.bs);
  };

  // ---- tile loads into registers: piece v = i * 256 + tid of the tile is key
  //      v / V8, head-dim piece v % V8; K and V share the slot arithmetic
  constexpr int KPI = kPW * 64 / V8;  // keys covered by one i
  v8s kreg[LPT], vreg[LPT];
  auto load_tile = [&](int tile) {
    const int kbase = tile * kKT;
    const int d8 = tid & (V8 - 1);
    const int kl = tid >> V8_SHIFT;
    if (kbase + kKT <= L) {
#pragma unroll
      for (int i = 0; i < LPT; ++i) {
        int64_t slot;
        if constexpr (KPI <= 16) {
          // the KPI keys of step i lie in one cache block: uniform block id
          const int j0 = kbase + i * KPI;
          const int q = div_magic(j0, a.bs_magic);
          slot = (int64_t)btab[q] * a.bs + (j0 - q * a.bs) + kl;
        } else {
          slot = slot_of(kbase + i * KPI + kl);
        }
        const int64_t off = slot * row_stride + d8 * 8;
        kreg[i] = *reinterpret_cast<const v8s*>(kc + off);
        vreg[i] = *reinterpret_cast<const v8s*>(vc + off);
      }
    } else {
      const v8s z = {0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll
      for (int i = 0; i < LPT; ++i) {
        const int j = kbase + i * KPI + kl;
        kreg[i] = z;
        vreg[i] = z;
        if (j < L) {
          const int64_t off = slot_of(j) * row_stride + d8 * 8;
          kreg[i] = *reinterpret_cast<const v8s*>(kc + off);
          vreg[i] = *reinterpret_cast<const v8s*>(vc + off);
        }
      }
    }
  };
  auto store_tile = [&](int stage) {
    uint16_t* ks = reinterpret_cast<uint16_t*>(smem + stage * kStageBytes<D>);
    uint16_t* vs = ks + kKT * KP;
#pragma unroll
    for (int i = 0; i < LPT; ++i) {
      const int v = i * kPW * 64 + tid;
      const int off = (v >> V8_SHIFT) * KP + (v & (V8 - 1)) * 8;
      *reinterpret_cast<v8s*>(ks + off) = kreg[i];
      *reinterpret_cast<v8s*>(vs + off) = vreg[i];
    }
  };

  float m_run = kNegInf;   // reference maximum of the row (log2 units)
  float l_run = 0.0f;      // this lane's half of the row sum
  v16f oacc[DC];
#pragma unroll
  for (int dc = 0; dc < DC; ++dc)
#pragma unroll
    for (int e = 0; e < 16; ++e) oacc[dc][e] = 0.0f;

  if (t_begin < t_end) {
    load_tile(t_begin);
    store_tile(0);
  }
  // every global load so far (Q included) has landed: keeps the compiler
  // from waiting on the next-tile prefetch at the first use of Q in the loop
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
  __syncthreads();

  // logits z: raw score (no softcap / ALiBi) scaled by cz in the exponent, or
  // the finished log2-unit logit with cz = 1
  const float cz = (SOFTCAP || ALIBI) ? 1.0f : a.scale_log2;

  for (int tile = t_begin; tile < t_end; ++tile) {
    const int stage = (tile - t_begin) & 1;
    const bool more = tile + 1 < t_end;
    if (more) load_tile(tile + 1);

    const int kbase = tile * kKT;
    bool active = w_rows;
    if (a.causal) active = active && kbase <= w_pmax;
    if (a.window_left >= 0) active = active && kbase + kKT - 1 >= w_pmin - a.window_left;

    if (active) {
      const uint16_t* ks = reinterpret_cast<const uint16_t*>(smem + stage * kStageBytes<D>);
      const uint16_t* vs = ks + kKT * KP;

      // ---- S^T = K Q^T for keys kbase + [0, 32) and [32, 64)
      v16f sacc[2];
#pragma unroll
      for (int h2 = 0; h2 < 2; ++h2) {
#pragma unroll
        for (int e = 0; e < 16; ++e) sacc[h2][e] = 0.0f;
        const uint16_t* krow = ks + (h2 * 32 + r32) * KP + 8 * g2;
#pragma unroll
        for (int kk = 0; kk < KQ; ++kk)
          sacc[h2] = T::mfma32x32x16(*reinterpret_cast<const v8s*>(krow + 16 * kk), qf[kk],
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

      // ---- lazy rescale: move the reference only when the max grew a lot
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

      float psum = 0.0f;
      v8s pb[4];
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        float pv[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          pv[e] = fast_exp2(fmaf(sacc[s >> 1][8 * (s & 1) + e], cz, neg_m));
          psum += pv[e];
        }
        u32x4 w = {T::pack2(pv[0], pv[1]), T::pack2(pv[2], pv[3]), T::pack2(pv[4], pv[5]),
                   T::pack2(pv[6], pv[7])};
        pb[s] = __builtin_bit_cast(v8s, w);
      }
      l_run += psum;

      // ---- O^T += V^T P^T; the A operand of step s holds V[16s + 4*g2 + [0,4)][d] and
      //      V[16s + 8 + 4*g2 + [0,4)][d] for d = dc*32 + r32 (two transpose reads)
      const uint16_t* vbase = vs + (4 * g2 + ((lane & 15) >> 2)) * KP + 16 * ((lane >> 4) & 1) +
                              4 * (lane & 3);
#pragma unroll
      for (int s = 0; s < 4; ++s) {
#pragma unroll
        for (int dc = 0; dc < DC; ++dc) {
          const uint16_t* p0 = vbase + (16 * s) * KP + dc * 32;
          const v4s lo = lds_read_tr16(p0);
          const v4s hi = lds_read_tr16(p0 + 8 * KP);
          const v8s av = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
          oacc[dc] = T::mfma32x32x16(av, pb[s], oacc[dc]);
        }
      }
    }

    if (more) store_tile(stage ^ 1);
    __syncthreads();
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
  const int ntiles = (max_seqlen_q + args.tok_per_tile - 1) / args.tok_per_tile;
  if (ntiles == 0) return 0;
  const dim3 grid(args.Hkv, args.B, ntiles);
  hipLaunchKernelGGL((prefill_kernel<T, D, FEAT>), grid, dim3(kPW * 64), prefill_lds_bytes<D>(),
                     stream, args);
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
  a.tok_per_tile = kRows / a.G;
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
