// paged_attn_decode: one query token per sequence over the paged KV cache,
// optionally split along the keys (Aphrodite flash_attn.py,
// FlashAttentionImpl.forward, flash_attn_with_kvcache decode; vLLM
// flash_attn.py (e2f56c3), FlashAttentionMetadataBuilder num_splits and its
// intermediate buffers).
//
// Work item = (kv head g, sequence b, split).  The G = Hq / Hkv query heads
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
  uint32_t bs_magic;    // ceil(2^32 / bs)
  float scale_log2;     // scale * log2(e)
  float scale_over_cap; // scale / softcap
  float cap_log2;       // softcap * log2(e)
  int window_left;      // -1 = none
  const float* alibi;   // nullable
};

enum { kSoftcap = 1, kAlibi = 2 };
constexpr float kTau = 8.0f;  // lazy-rescale threshold (log2 units)

// LDS: per-wave V slabs of 16 rows (pitch D + 16 elements: the 32-byte pad
// spreads the 16 rows a transpose read touches over all banks), reused after
// the key loop for the cross-wave combine: [wave][head j < G][m, l, O[0..D)].
template <int D>
constexpr int kVPitch = D + 16;
template <int D>
constexpr size_t decode_lds_bytes(int G) {
  const size_t v = (size_t)kWaves * 16 * kVPitch<D> * 2;
  const size_t c = (size_t)kWaves * G * (D + 2) * 4;
  return v > c ? v : c;
}

template <typename T, int D, int FEAT>
__global__ __launch_bounds__(kWaves * 64) void decode_kernel(DecodeArgs a) {
  constexpr bool SOFTCAP = FEAT & kSoftcap;
  constexpr bool ALIBI = FEAT & kAlibi;
  constexpr int KK = D / 32;   // QK mfma steps along D
  constexpr int DC = D / 16;   // PV output chunks of 16 rows of D
  constexpr int P = kVPitch<D>;
  extern __shared__ __attribute__((aligned(16))) char smem[];

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int r16 = lane & 15;   // key row of the K piece / head column of the tile
  const int c4 = lane >> 4;    // which quarter: keys 4*c4..4*c4+3 of S^T, D piece of K

  const int g = blockIdx.x % a.Hkv;
  const int rest = blockIdx.x / a.Hkv;
  const int b = rest % a.B;
  const int split = rest / a.B;

  const int L = a.seq_lens[b];
  const int pos = L - 1;
  const int per = (L + a.S - 1) / a.S;
  const int chunk = ((per + a.bs - 1) / a.bs) * a.bs;
  const int lo = min(split * chunk, L);
  const int hi = min(lo + chunk, L);
  const int lo_vis = a.window_left >= 0 ? max(lo, pos - a.window_left) : lo;
  const int t_begin = lo_vis >> 4;
  const int t_end = (hi + 15) >> 4;

  const int head = g * a.G + r16;  // query head of this lane's column
  const bool col_ok = r16 < a.G;
  float slope_log2 = 0.0f;
  if constexpr (ALIBI) slope_log2 = col_ok ? a.alibi[head] * kLog2e : 0.0f;

  // Q^T as the B operand: column r16, D elements kk*32 + c4*8 .. +8
  v8s qf[KK];
  {
    const uint16_t* qrow = a.q + ((int64_t)b * a.Hq + head) * D + c4 * 8;
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
      v8s z = {0, 0, 0, 0, 0, 0, 0, 0};
      qf[kk] = col_ok ? *reinterpret_cast<const v8s*>(qrow + kk * 32) : z;
    }
  }

  const int32_t* btab = a.block_table + (int64_t)b * a.bt_stride;
  const int64_t row_stride = (int64_t)a.Hkv * D;  // elements between consecutive slots

  struct Frag {
    v8s k[KK];
    v8s v[KK];
  };
  auto load_tile = [&](int tile, Frag& f) {
    const int j0 = tile << 4;
    const int q = div_magic(j0, a.bs_magic);
    const int64_t slot = (int64_t)btab[q] * a.bs + (j0 - q * a.bs) + r16;
    const int64_t off = slot * row_stride + (int64_t)g * D + c4 * 8;
    const uint16_t* kp = a.kc + off;
    const uint16_t* vp = a.vc + off;
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
      f.k[kk] = *reinterpret_cast<const v8s*>(kp + kk * 32);
      f.v[kk] = *reinterpret_cast<const v8s*>(vp + kk * 32);
    }
  };

  float m_run = kNegInf;  // running max (base-2 units) of column r16
  float l_run = 0.0f;     // this lane's share of the running sum
  v4f o[DC];
#pragma unroll
  for (int dc = 0; dc < DC; ++dc) o[dc] = v4f{0.f, 0.f, 0.f, 0.f};

  uint16_t* vs = reinterpret_cast<uint16_t*>(smem) + wave * 16 * P;

  Frag cur, nxt;
  int tile = t_begin + wave;
  if (tile < t_end) load_tile(tile, cur);
  for (; tile < t_end; tile += kWaves) {
    const int tn = tile + kWaves;
    if (tn < t_end) load_tile(tn, nxt);

    const int j0 = tile << 4;
    // ---- scores S^T[key j0 + 4*c4 + e][head r16], in log2 units
    v4f s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) s = T::mfma16x16x32(cur.k[kk], qf[kk], s);
    float x[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int key = j0 + 4 * c4 + e;
      float v;
      if constexpr (SOFTCAP) v = a.cap_log2 * tanh_f32(s[e] * a.scale_over_cap);
      else v = s[e] * a.scale_log2;
      if constexpr (ALIBI) v -= slope_log2 * static_cast<float>(pos - key);
      x[e] = (key >= lo_vis && key < hi) ? v : kNegInf;
    }
    // ---- online softmax over the 16 keys of this tile, per head column;
    //      the reference max only moves when it grows by more than 2^8
    float mx = fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3]));
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
    float pe[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) pe[e] = fast_exp2(x[e] - m_use);
    l_run += (pe[0] + pe[1]) + (pe[2] + pe[3]);
    u32x2 pw = {T::pack2(pe[0], pe[1]), T::pack2(pe[2], pe[3])};
    const v4s pb = __builtin_bit_cast(v4s, pw);

    // ---- V tile -> LDS (row r16); rows outside [lo_vis, hi) become zero so
    //      stale or poisoned cache contents never reach the accumulator
    {
      const int key = j0 + r16;
      const bool row_ok = key >= lo_vis && key < hi;
      uint16_t* dst = vs + r16 * P + c4 * 8;
#pragma unroll
      for (int kk = 0; kk < KK; ++kk) {
        v8s z = {0, 0, 0, 0, 0, 0, 0, 0};
        *reinterpret_cast<v8s*>(dst + kk * 32) = row_ok ? cur.v[kk] : z;
      }
    }
    wave_lds_sync();
    // ---- O^T[d][head] += V^T[d][key] P^T[key][head]; lane group c4 reads
    //      V[4*c4 + e][dc*16 + r16] for e = 0..3 with one transpose read
    {
      const uint16_t* vb = vs + (4 * c4 + (r16 >> 2)) * P + 4 * (r16 & 3);
#pragma unroll
      for (int dc = 0; dc < DC; ++dc) o[dc] = T::mfma16x16x16(lds_read_tr16(vb + dc * 16), pb, o[dc]);
    }
    wave_lds_sync();
    cur = nxt;
  }

  // ---- combine the waves: lane holds O^T[d = dc*16 + 4*c4 + e][head r16]
  float l_tot = l_run + shfl_xor(l_run, 16);
  l_tot += shfl_xor(l_tot, 32);
  __syncthreads();  // every wave is done with its V slab
  float* comb = reinterpret_cast<float*>(smem);  // [wave][G][D + 2]: m, l, O[D]
  constexpr int CP = D + 2;
  if (col_ok) {
    float* row = comb + (wave * a.G + r16) * CP;
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
  const bool split_out = a.S > 1;
  for (int idx = threadIdx.x; idx < a.G * D; idx += kWaves * 64) {
    const int j = idx / D;
    const int d = idx - j * D;
    float M = kNegInf;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) M = fmaxf(M, comb[(w * a.G + j) * CP]);
    float num = 0.f, den = 0.f;
    if (M != kNegInf) {
#pragma unroll
      for (int w = 0; w < kWaves; ++w) {
        const float* row = comb + (w * a.G + j) * CP;
        const float f = fast_exp2(row[0] - M);
        den += f * row[1];
        num += f * row[2 + d];
      }
    }
    const float val = den > 0.f ? num / den : 0.f;
    const int h = g * a.G + j;
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

template <typename T, int D, int FEAT>
int launch_d(const DecodeArgs& args, hipStream_t stream) {
  const int64_t grid = (int64_t)args.Hkv * args.B * args.S;
  hipLaunchKernelGGL((decode_kernel<T, D, FEAT>), dim3(static_cast<unsigned>(grid)),
                     dim3(kWaves * 64), decode_lds_bytes<D>(args.G), stream, args);
  return hipGetLastError() == hipSuccess ? 0 : -3;
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
