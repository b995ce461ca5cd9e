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
// cross-lane step pairs lane l with l ^ 32), and the fp32 probabilities of
// S^T become the B operand of the PV product in registers, without moving.
//
// K/V tiles are gathered block by block through the block table into
// registers one tile ahead, then stored to a double-buffered LDS stage:
// K row-major (16-byte rows pieces), V transposed (one LDS row per head
// dimension) so the PV A operand is two 8-byte reads per lane.  Keys at or
// past the sequence end are never loaded (zero in LDS), so block-table
// padding and poisoned tails are never touched.
#include "common.h"
#include "launch.h"

namespace pa {

namespace {

constexpr int kPW = 4;      // waves per workgroup
constexpr int kRows = 128;  // MFMA rows per workgroup
constexpr int kKT = 64;     // keys per tile

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
  float scale, scale_log2, softcap;
  int causal, window_left;
  const float* alibi;
};

template <int D>
constexpr int kKPitch = D + 8;      // K rows: 16-byte pad
constexpr int kVtPitch = kKT + 4;   // V^T rows: 8-byte pad
template <int D>
constexpr int kStageBytes = (kKT * kKPitch<D> + D * kVtPitch) * 2;
template <int D>
constexpr size_t prefill_lds_bytes() { return 2 * (size_t)kStageBytes<D>; }

template <typename T, int D>
__global__ __launch_bounds__(kPW * 64) void prefill_kernel(PrefillArgs a) {
  constexpr int KQ = D / 16;        // QK mfma steps along D
  constexpr int DC = D / 32;        // PV output chunks of 32 head dims
  constexpr int V8 = D / 8;         // 16-byte pieces per row
  constexpr int LPT = kKT * V8 / (kPW * 64);  // pieces per thread per tile (K and V each)
  constexpr int KP = kKPitch<D>;
  constexpr int VP = kVtPitch;
  extern __shared__ __attribute__((aligned(16))) char smem[];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
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
  const int tok_end = min(nq, tok0 + a.tok_per_tile);
  const int p_first = ctx + tok0;
  const int p_last = ctx + tok_end - 1;
  const int k_hi = a.causal ? min(L, p_last + 1) : L;
  const int k_lo = a.window_left >= 0 ? max(0, p_first - a.window_left) : 0;
  const int t_begin = k_lo / kKT;
  const int t_end = (k_hi + kKT - 1) / kKT;

  // this lane's query row
  const int row = wave * 32 + r32;
  const int tk = row / a.G;
  const int hh = row - tk * a.G;
  const bool row_ok = row < a.tok_per_tile * a.G && tok0 + tk < nq;
  const int pos = ctx + tok0 + tk;
  const int head = g * a.G + hh;
  const float slope_log2 = (a.alibi != nullptr && row_ok) ? a.alibi[head] * kLog2e : 0.0f;

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
  const int64_t head_off = (int64_t)g * D;

  // ---- tile loads into registers
  v8s kreg[LPT], vreg[LPT];
  auto load_tile = [&](int tile) {
    const int kbase = tile * kKT;
#pragma unroll
    for (int i = 0; i < LPT; ++i) {
      const int v = i * kPW * 64 + tid;
      const int key = v / V8;
      const int d8 = v - key * V8;
      const int j = kbase + key;
      v8s z = {0, 0, 0, 0, 0, 0, 0, 0};
      kreg[i] = z;
      if (j < L) {
        const int64_t slot = (int64_t)btab[j / a.bs] * a.bs + (j % a.bs);
        kreg[i] = *reinterpret_cast<const v8s*>(a.kc + slot * row_stride + head_off + d8 * 8);
      }
    }
    {
      const int key = tid % kKT;
      const int j = kbase + key;
      int64_t base = -1;
      if (j < L) base = ((int64_t)btab[j / a.bs] * a.bs + (j % a.bs)) * row_stride + head_off;
#pragma unroll
      for (int i = 0; i < LPT; ++i) {
        const int d8 = tid / kKT + (kPW * 64 / kKT) * i;
        v8s z = {0, 0, 0, 0, 0, 0, 0, 0};
        vreg[i] = base >= 0 ? *reinterpret_cast<const v8s*>(a.vc + base + d8 * 8) : z;
      }
    }
  };
  auto store_tile = [&](int stage) {
    uint16_t* ks = reinterpret_cast<uint16_t*>(smem + stage * kStageBytes<D>);
    uint16_t* vt = ks + kKT * KP;
#pragma unroll
    for (int i = 0; i < LPT; ++i) {
      const int v = i * kPW * 64 + tid;
      const int key = v / V8;
      const int d8 = v - key * V8;
      *reinterpret_cast<v8s*>(ks + key * KP + d8 * 8) = kreg[i];
    }
    const int key = tid % kKT;
#pragma unroll
    for (int i = 0; i < LPT; ++i) {
      const int d8 = tid / kKT + (kPW * 64 / kKT) * i;
#pragma unroll
      for (int e = 0; e < 8; ++e) vt[(d8 * 8 + e) * VP + key] = static_cast<uint16_t>(vreg[i][e]);
    }
  };

  float m_run = kNegInf;
  float l_run = 0.0f;
  v16f oacc[DC];
#pragma unroll
  for (int dc = 0; dc < DC; ++dc)
#pragma unroll
    for (int e = 0; e < 16; ++e) oacc[dc][e] = 0.0f;

  if (t_begin < t_end) {
    load_tile(t_begin);
    store_tile(0);
  }
  __syncthreads();

  for (int tile = t_begin; tile < t_end; ++tile) {
    const int stage = (tile - t_begin) & 1;
    const bool more = tile + 1 < t_end;
    if (more) load_tile(tile + 1);

    const uint16_t* ks = reinterpret_cast<const uint16_t*>(smem + stage * kStageBytes<D>);
    const uint16_t* vt = ks + kKT * KP;
    const int kbase = tile * kKT;

    // ---- S^T = K Q^T for keys kbase + [0, 32) and [32, 64)
    v16f sacc[2];
#pragma unroll
    for (int h2 = 0; h2 < 2; ++h2) {
#pragma unroll
      for (int e = 0; e < 16; ++e) sacc[h2][e] = 0.0f;
      const uint16_t* krow = ks + (h2 * 32 + r32) * KP + 8 * g2;
#pragma unroll
      for (int kk = 0; kk < KQ; ++kk)
        sacc[h2] = T::mfma32x32x16(*reinterpret_cast<const v8s*>(krow + 16 * kk), qf[kk], sacc[h2]);
    }

    // ---- scores -> base-2 logits with masks; lane holds keys
    //      kbase + 32*h2 + 8*(e/4) + 4*g2 + e%4 of its row
    float x[2][16];
    float mx = kNegInf;
#pragma unroll
    for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int key = kbase + 32 * h2 + 8 * (e >> 2) + 4 * g2 + (e & 3);
        float v;
        if (a.softcap > 0.f)
          v = a.softcap * tanh_f32(sacc[h2][e] * a.scale / a.softcap) * kLog2e;
        else
          v = sacc[h2][e] * a.scale_log2;
        const int dist = pos - key;
        v -= slope_log2 * static_cast<float>(dist < 0 ? -dist : dist);
        bool vis = key < L;
        if (a.causal) vis = vis && key <= pos;
        if (a.window_left >= 0) vis = vis && key >= pos - a.window_left;
        v = vis ? v : kNegInf;
        x[h2][e] = v;
        mx = fmaxf(mx, v);
      }
    mx = fmaxf(mx, shfl_xor(mx, 32));
    const float m_new = fmaxf(m_run, mx);
    const float m_use = m_new == kNegInf ? 0.0f : m_new;
    const float alpha = fast_exp2(m_run - m_use);
    m_run = m_new;
    float psum = 0.0f;
    v8s pb[4];
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      float pv[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        pv[e] = fast_exp2(x[s >> 1][8 * (s & 1) + e] - m_use);
        psum += pv[e];
      }
      u32x4 w = {T::pack2(pv[0], pv[1]), T::pack2(pv[2], pv[3]), T::pack2(pv[4], pv[5]),
                 T::pack2(pv[6], pv[7])};
      pb[s] = __builtin_bit_cast(v8s, w);
    }
    l_run = l_run * alpha + psum;
#pragma unroll
    for (int dc = 0; dc < DC; ++dc) oacc[dc] *= alpha;

    // ---- O^T += V^T P^T; keys of step s: 16s + 4*g2 + [0,4) and 16s + 8 + 4*g2 + [0,4)
#pragma unroll
    for (int s = 0; s < 4; ++s) {
#pragma unroll
      for (int dc = 0; dc < DC; ++dc) {
        const uint16_t* vrow = vt + (dc * 32 + r32) * VP + 16 * s + 4 * g2;
        const u32x2 lo = *reinterpret_cast<const u32x2*>(vrow);
        const u32x2 hi = *reinterpret_cast<const u32x2*>(vrow + 8);
        const u32x4 w = {lo[0], lo[1], hi[0], hi[1]};
        oacc[dc] = T::mfma32x32x16(__builtin_bit_cast(v8s, w), pb[s], oacc[dc]);
      }
    }

    if (more) store_tile(stage ^ 1);
    __syncthreads();
  }

  // ---- epilogue: lane holds O^T[d = dc*32 + 8*(e/4) + 4*g2 + e%4][row]
  const float l_tot = l_run + shfl_xor(l_run, 32);
  if (!row_ok) return;
  const float inv = l_tot > 0.f ? 1.0f / l_tot : 0.0f;
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
    a.lse[(int64_t)head * a.total_q + qrow] = l_tot > 0.f ? (m_run + __log2f(l_tot)) * kLn2 : kNegInf;
}

template <typename T, int D>
int launch_p(const PrefillArgs& args, int max_seqlen_q, hipStream_t stream) {
  const int ntiles = (max_seqlen_q + args.tok_per_tile - 1) / args.tok_per_tile;
  if (ntiles == 0) return 0;
  const dim3 grid(args.Hkv, args.B, ntiles);
  hipLaunchKernelGGL((prefill_kernel<T, D>), grid, dim3(kPW * 64), prefill_lds_bytes<D>(), stream,
                     args);
  return hipGetLastError() == hipSuccess ? 0 : -3;
}

template <typename T, int D>
void set_lds_limit() {
  static bool done = false;
  if (!done) {
    done = hipFuncSetAttribute(reinterpret_cast<const void*>(&prefill_kernel<T, D>),
                               hipFuncAttributeMaxDynamicSharedMemorySize,
                               static_cast<int>(prefill_lds_bytes<D>())) == hipSuccess;
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
  a.tok_per_tile = kRows / a.G;
  a.scale = p.scale;
  a.scale_log2 = p.scale * kLog2e;
  a.softcap = p.softcap;
  a.causal = p.causal;
  a.window_left = p.window_left;
  a.alibi = p.alibi_slopes;
  const bool bf = p.dtype == kBF16;
  switch (p.head_size) {
    case 64:
      if (bf) { set_lds_limit<BF16, 64>(); return launch_p<BF16, 64>(a, p.max_seqlen_q, stream); }
      set_lds_limit<F16, 64>();
      return launch_p<F16, 64>(a, p.max_seqlen_q, stream);
    case 128:
      if (bf) { set_lds_limit<BF16, 128>(); return launch_p<BF16, 128>(a, p.max_seqlen_q, stream); }
      set_lds_limit<F16, 128>();
      return launch_p<F16, 128>(a, p.max_seqlen_q, stream);
    default:
      if (bf) { set_lds_limit<BF16, 256>(); return launch_p<BF16, 256>(a, p.max_seqlen_q, stream); }
      set_lds_limit<F16, 256>();
      return launch_p<F16, 256>(a, p.max_seqlen_q, stream);
  }
}

}  // namespace pa
