// Mixed-precision paged decode attention for the OSCAR INT2 KV cache (gfx950).
//
// Read path of the OSCAR pages ([IT] 2.2.B, [ES] "El sistema de servicio",
// read path): the INT2 history is unpacked and dequantised inside the attention
// kernel; sink and recent tokens are read as bf16.  Instead of rotating every
// token back, the rotation is undone algebraically:
//     q . (x_rot R^T) = (q R) . x_rot      for keys,
//     sum_t p_t x_rot,t R^T = (sum_t p_t x_rot,t) R^T   for values,
// so q R_K is formed once per query (prologue) and R_V^T once per output row
// (combine).
//
// Kernels
//   decode_prologue  per (request, KV head): q R_K for the g query heads of the
//                    group, turned into MFMA operands.
//   decode_main      per (request, KV head, split): one wavefront streams its
//                    share of pages, two pages (32 tokens) per iteration.
//   decode_combine   per (request, KV head): log-sum-exp merge of the splits,
//                    R_V^T on the INT2 part, normalisation.
//
// INT2 logits on MFMA (v_mfma_i32_16x16x64_i8, exact integer accumulation):
//   q~ = (q R_K) log2(e)/sqrt(d) is held as the fixed-point integer
//   Q = rint(q~ 2^sq) (|Q| < 2^22 per head), split into three balanced int8
//   digits Q = d0 2^16 + d1 2^8 + d2.  A = the 2-bit codes as int8 bytes,
//   B = the digits, block-diagonal over channel groups: column (h, gamma) only
//   sees channels of group gamma, so C[t, (h, gamma)] = sum_{j in gamma} Q_hj c_tj
//   exactly.  With the group sum Qbar = sum_{j in gamma} Q_hj,
//     sum_j Q_j (z + c_j s) = (s/2) (2C - 3 Qbar) + (z + 1.5 s) Qbar,
//   where 2C - 3 Qbar = sum_j Q_j (2 c_j - 3) is formed exactly in int32, so
//   the large, nearly cancelling terms s C and z Qbar are never rounded.
// INT2 values on MFMA:
//   A = P'[(h, gamma), t] = p_ht s_t,gamma 2^sp 2^-2r (hi + lo fp16),
//   B = centred V codes (2c - 3) 2^(2r-24) as exact fp16 subnormals
//       (channel-major words make a lane's 8 tokens of one channel a single
//       16-bit word; one packed fp16 fma centres them),
//   acc[(h, gamma), j] for j in group gamma; the midpoint term
//   sum_t p_ht (z + 1.5 s)_t,gamma is accumulated on the VALU.  Centring keeps
//   both sums free of the large cancelling parts sum p z and sum p s c.
// bf16 tokens use v_mfma_f32_16x16x32_bf16 with the unrotated query (exact
// products) and P split into bf16 hi + mid + lo.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <cmath>

#include "oscar_internal.h"

namespace oscar {
namespace {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2eOverSqrtD = 0.12751743074133604f;  // log2(e) / sqrt(128)
constexpr float kNegInf = -__builtin_huge_valf();
constexpr int kPartialStride = 2 + kHeadDim;

__device__ __forceinline__ f32x4 mfma_f16(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b), c, 0,
                                                0, 0);
}
__device__ __forceinline__ i32x4 mfma_i8(u32x4 a, u32x4 b, i32x4 c) {
  return __builtin_amdgcn_mfma_i32_16x16x64_i8(__builtin_bit_cast(i32x4, a), __builtin_bit_cast(i32x4, b), c, 0, 0,
                                               0);
}
__device__ __forceinline__ f32x4 mfma_bf16(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c,
                                                 0, 0, 0);
}

__device__ __forceinline__ float half_lo(uint32_t w) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)(w & 0xffffu));
}
__device__ __forceinline__ float half_hi(uint32_t w) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)(w >> 16));
}
__device__ __forceinline__ uint32_t pack_f16(float lo, float hi) {
  return (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)lo) |
         ((uint32_t)__builtin_bit_cast(uint16_t, (_Float16)hi) << 16);
}
// fp32 -> bf16 bits, nearest-even (finite inputs)
__device__ __forceinline__ uint32_t bf16_bits(float x) {
  uint32_t u = __builtin_bit_cast(uint32_t, x);
  return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}
__device__ __forceinline__ float bf16_val(uint32_t b) { return __builtin_bit_cast(float, b << 16); }

// butterfly sum over the NG lanes of a channel-group set (lanes differ in the low bits)
template <int NG>
__device__ __forceinline__ float group_sum(float x) {
  x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0xB1, 0xF, 0xF, false));
  if constexpr (NG == 4)
    x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x4E, 0xF, 0xF, false));
  return x;
}
__device__ __forceinline__ float max_across_quads(float x) {
  x = fmaxf(x, __shfl_xor(x, 16));
  x = fmaxf(x, __shfl_xor(x, 32));
  return x;
}
__device__ __forceinline__ float sum_across_quads(float x) {
  x += __shfl_xor(x, 16);
  x += __shfl_xor(x, 32);
  return x;
}

__device__ __forceinline__ const uint8_t* block_ptr(const uint8_t* base, int64_t page, int n_kv, int kv,
                                                    int bytes) {
  return base + ((page * n_kv + kv) * (int64_t)bytes);
}

// ---------------------------------------------------------------------------
// prologue: q R_K operands
// ---------------------------------------------------------------------------
// Words per (request, KV head): B digits ((((ct*3 + digit)*2 + kstep)*64 + lane)*4 + reg),
// then aux floats [1 + 32*CT]: logit factor 2^-sq / 2, per column 2*Qbar (float),
// per column -3*Qbar (int32 bits).
template <int NG, int CT>
__global__ __launch_bounds__(128) void decode_prologue(DecodeParams p) {
  const int bk = blockIdx.x;
  const int b = bk / p.n_kv, kv = bk % p.n_kv;
  const int j = threadIdx.x;
  constexpr int G = kHeadDim / NG;
  __shared__ float qs[16][kHeadDim];
  __shared__ int qi[16][kHeadDim];
  __shared__ float red[4];
  const int g = p.g;
  for (int h = 0; h < g; ++h)
    qs[h][j] = bf16_val(p.q[((int64_t)b * p.n_q + kv * g + h) * kHeadDim + j]);
  __syncthreads();
  const float* R = p.r_k + (int64_t)kv * kHeadDim * kHeadDim;
  float qt[16];
  float mx = 0.f;
  for (int h = 0; h < g; ++h) {
    float acc = 0.f;
    for (int i = 0; i < kHeadDim; ++i) acc = fmaf(qs[h][i], R[i * kHeadDim + j], acc);
    qt[h] = acc * kLog2eOverSqrtD;
    mx = fmaxf(mx, fabsf(qt[h]));
  }
  for (int off = 32; off >= 1; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off));
  if ((j & 63) == 0) red[j >> 6] = mx;
  __syncthreads();
  mx = fmaxf(red[0], red[1]);
  // 2^sq brings the largest |q~| to [2^21, 2^22)
  int sq = 0;
  if (mx > 0.f && mx < __builtin_huge_valf()) {
    int e;
    frexpf(mx, &e);  // mx in [2^(e-1), 2^e)
    sq = 22 - e;
  }
  for (int h = 0; h < g; ++h) qi[h][j] = (int)rintf(ldexpf(qt[h], sq));
  __syncthreads();
  float* aux = p.qaux + (int64_t)bk * (1 + 32 * CT);
  if (j == 0) aux[0] = ldexpf(0.5f, -sq);
  if (j < 16 * CT) {
    const int h = j / NG, gam = j % NG;
    int sum = 0;
    if (h < g)
      for (int c = gam * G; c < (gam + 1) * G; ++c) sum += qi[h][c];
    aux[1 + j] = 2.0f * (float)sum;
    aux[1 + 16 * CT + j] = __builtin_bit_cast(float, -3 * sum);
  }
  uint32_t* qb = p.qb + (int64_t)bk * CT * 3 * 2 * 64 * 4;
  for (int w = j; w < CT * 3 * 2 * 64 * 4; w += 128) {
    const int reg = w & 3, lane = (w >> 2) & 63, ks = (w >> 8) & 1, rest = w >> 9;
    const int digit = rest % 3, ct = rest / 3;
    const int ln = lane & 15, qd = lane >> 4;
    const int col = 16 * ct + ln, h = col / NG, gam = col % NG;
    uint32_t word = 0;
    for (int byte = 0; byte < 4; ++byte) {
      const int ch = 32 * qd + 16 * ks + 4 * byte + reg;
      int dv = 0;
      if (h < g && ch / G == gam) {
        const int q = qi[h][ch];
        const int d2 = ((q + 128) & 255) - 128;
        const int q1 = (q - d2) >> 8;
        const int d1 = ((q1 + 128) & 255) - 128;
        const int d0 = (q1 - d1) >> 8;
        dv = digit == 0 ? d0 : (digit == 1 ? d1 : d2);
      }
      word |= (uint32_t)(dv & 0xff) << (8 * byte);
    }
    qb[w] = word;
  }
}

// ---------------------------------------------------------------------------
// main kernel: INT2 work item
// ---------------------------------------------------------------------------
template <int NG, int CT, bool EDGE>
__device__ __forceinline__ void int2_pair(const DecodeParams& p, const uint8_t* blk0, const uint8_t* blk1,
                                          int lp0, int p_end, int lo, int hi, const u32x4 (&bq)[CT][3][2],
                                          const float (&qbar2)[CT], const int (&qneg3)[CT], float kfac,
                                          float pscale, float (&m_run)[CT],
                                          float (&l_run)[CT], float (&zsum)[CT], f32x4 (&acc)[CT][8]) {
  constexpr Int2Layout L{NG};
  const int lane = threadIdx.x, ln = lane & 15, qd = lane >> 4;
  const int a = qd & 1, gam = ln % NG;
  // A operand rows (tokens) of the two QK tiles
  const uint8_t* bk = (ln >> 3) ? blk1 : blk0;
  const int tokA = 8 * ((ln >> 2) & 1) + (ln & 3);
  const u32x2 ka0 = *(const u32x2*)(bk + L.k_codes() + tokA * 32 + 8 * qd);
  const u32x2 ka1 = *(const u32x2*)(bk + L.k_codes() + (tokA + 4) * 32 + 8 * qd);
  // this lane's C rows / PV k-range: page qd>>1, tokens 8a + 4*tile + r
  const uint8_t* bq_ = (qd >> 1) ? blk1 : blk0;
  const u32x4 ksz0 = *(const u32x4*)(bq_ + L.k_sz() + (gam * 16 + 8 * a) * 4);
  const u32x4 ksz1 = *(const u32x4*)(bq_ + L.k_sz() + (gam * 16 + 8 * a + 4) * 4);
  const u32x4 vw = *(const u32x4*)(bq_ + L.v_codes() + (a * 128 + 8 * ln) * 2);
  const u32x4 vsz0 = *(const u32x4*)(bq_ + L.v_sz() + (gam * 16 + 8 * a) * 4);
  const u32x4 vsz1 = *(const u32x4*)(bq_ + L.v_sz() + (gam * 16 + 8 * a + 4) * 4);

  // ---- QK: exact integer sums per (token, (h, gamma)) ----
  // A register k of K-step ks holds, byte b, the code of channel 32qd + 16ks + 4b + k.
  i32x4 c[2][CT];
  const uint32_t kd[2][2] = {{ka0[0], ka0[1]}, {ka1[0], ka1[1]}};
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    i32x4 cd[CT][3];
#pragma unroll
    for (int ct = 0; ct < CT; ++ct)
#pragma unroll
      for (int d = 0; d < 3; ++d) cd[ct][d] = i32x4{0, 0, 0, 0};
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const uint32_t x = kd[t][ks];
      const u32x4 av = {x & 0x03030303u, (x >> 2) & 0x03030303u, (x >> 4) & 0x03030303u, (x >> 6) & 0x03030303u};
#pragma unroll
      for (int ct = 0; ct < CT; ++ct)
#pragma unroll
        for (int d = 0; d < 3; ++d) cd[ct][d] = mfma_i8(av, bq[ct][d][ks], cd[ct][d]);
    }
#pragma unroll
    for (int ct = 0; ct < CT; ++ct)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int cc = (cd[ct][0][r] * 256 + cd[ct][1][r]) * 256 + cd[ct][2][r];  // sum Q c
        c[t][ct][r] = 2 * cc + qneg3[ct];                                           // sum Q (2c - 3)
      }
  }
  // ---- logits (log2 domain) ----
  const int lp = lp0 + (qd >> 1);
  const int pos0 = lp * kPage + 8 * a;
  bool valid[2][4];
#pragma unroll
  for (int t = 0; t < 2; ++t)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      if constexpr (EDGE) {
        const int pos = pos0 + 4 * t + r;
        valid[t][r] = lp < p_end && pos >= lo && pos < hi;
      } else {
        valid[t][r] = true;
      }
    }
  float lg[2][CT][4];
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const u32x4 sz = t ? ksz1 : ksz0;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      float sv = half_lo(sz[r]), zv = half_hi(sz[r]);
      if constexpr (EDGE) {
        sv = valid[t][r] ? sv : 0.f;
        zv = valid[t][r] ? zv : 0.f;
      }
      const float mid = fmaf(1.5f, sv, zv);   // group midpoint z + 1.5 s (exact)
#pragma unroll
      for (int ct = 0; ct < CT; ++ct) {
        float x = fmaf(sv, (float)c[t][ct][r], mid * qbar2[ct]);
        x = group_sum<NG>(x) * kfac;
        lg[t][ct][r] = valid[t][r] ? x : kNegInf;
      }
    }
  }
  // ---- online softmax ----
  float pr[2][CT][4];
#pragma unroll
  for (int ct = 0; ct < CT; ++ct) {
    float mt = kNegInf;
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int r = 0; r < 4; ++r) mt = fmaxf(mt, lg[t][ct][r]);
    mt = max_across_quads(mt);
    const float m_new = fmaxf(m_run[ct], mt);
    if (__builtin_amdgcn_ballot_w64(m_new > m_run[ct])) {
      const float alpha = (m_new == kNegInf) ? 1.f : exp2f(m_run[ct] - m_new);
      l_run[ct] *= alpha;
      zsum[ct] *= alpha;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float ar = __shfl(alpha, 4 * qd + r);
#pragma unroll
        for (int kt = 0; kt < 8; ++kt) acc[ct][kt][r] *= ar;
      }
      m_run[ct] = m_new;
    }
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float e = exp2f(lg[t][ct][r] - m_run[ct]);
        pr[t][ct][r] = valid[t][r] ? e : 0.f;
        l_run[ct] += pr[t][ct][r];
      }
  }
  // ---- P' operands and zero-point term ----
  u32x4 pa[CT][2];
#pragma unroll
  for (int ct = 0; ct < CT; ++ct) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      float s0 = half_lo(vsz0[r]), z0 = half_hi(vsz0[r]);
      float s1 = half_lo(vsz1[r]), z1 = half_hi(vsz1[r]);
      if constexpr (EDGE) {
        s0 = valid[0][r] ? s0 : 0.f;
        z0 = valid[0][r] ? z0 : 0.f;
        s1 = valid[1][r] ? s1 : 0.f;
        z1 = valid[1][r] ? z1 : 0.f;
      }
      const float f = pscale * (1.0f / (float)(1 << (2 * r)));
      const float x0 = pr[0][ct][r] * s0 * f;
      const float x1 = pr[1][ct][r] * s1 * f;
      const float h0 = (float)(_Float16)x0, h1 = (float)(_Float16)x1;
      pa[ct][0][r] = pack_f16(h0, h1);
      pa[ct][1][r] = pack_f16(x0 - h0, x1 - h1);
      // value = (z + 1.5 s) + (c - 1.5) s: the midpoint part is summed here,
      // the centred codes go through the MFMA
      zsum[ct] = fmaf(pr[0][ct][r], fmaf(1.5f, s0, z0), zsum[ct]);
      zsum[ct] = fmaf(pr[1][ct][r], fmaf(1.5f, s1, z1), zsum[ct]);
    }
  }
  // ---- PV ----
#pragma unroll
  for (int kt = 0; kt < 8; ++kt) {
    const uint32_t w = (kt & 1) ? (vw[kt >> 1] >> 16) : (vw[kt >> 1] & 0xffffu);
    const uint32_t x = (w & 0xffu) | ((w & 0xff00u) << 8);
    // centred codes (2c - 3) 2^(2r-24), exact fp16 subnormals: 2 * (c 2^(2r-24)) - 3 2^(2r-24)
    u32x4 bv;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const f16x2 cv = __builtin_bit_cast(f16x2, x & (0x00030003u << (2 * r)));
      const _Float16 off = (_Float16)(-3.0f * (float)(1 << (2 * r)) * 5.9604644775390625e-08f);  // -3 2^(2r-24)
      bv[r] = __builtin_bit_cast(uint32_t, cv * (_Float16)2.0f + f16x2{off, off});
    }
#pragma unroll
    for (int ct = 0; ct < CT; ++ct) {
      acc[ct][kt] = mfma_f16(pa[ct][0], bv, acc[ct][kt]);
      acc[ct][kt] = mfma_f16(pa[ct][1], bv, acc[ct][kt]);
    }
  }
}

template <int NG, int CT>
__device__ void int2_item(const DecodeParams& p, int b, int kv, int split) {
  constexpr Int2Layout L{NG};
  const int lane = threadIdx.x, ln = lane & 15, qd = lane >> 4;
  const int T = p.ctx_lens[b];
  const int lo = p.sink;
  const int hi = T - p.recent;
  const int bk = b * p.n_kv + kv;
  float m_run[CT], l_run[CT], zsum[CT];
  f32x4 acc[CT][8];
#pragma unroll
  for (int ct = 0; ct < CT; ++ct) {
    m_run[ct] = kNegInf;
    l_run[ct] = 0.f;
    zsum[ct] = 0.f;
#pragma unroll
    for (int kt = 0; kt < 8; ++kt) acc[ct][kt] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  const float* aux = p.qaux + (int64_t)bk * (1 + 32 * CT);
  const float kfac = aux[0];
  float qbar2[CT];
  int qneg3[CT];
#pragma unroll
  for (int ct = 0; ct < CT; ++ct) {
    qbar2[ct] = aux[1 + 16 * ct + ln];
    qneg3[ct] = __builtin_bit_cast(int, aux[1 + 16 * CT + 16 * ct + ln]);
  }
  if (hi > lo && lo >= 0) {
    const int first = lo / kPage, last = (hi - 1) / kPage;
    const int n_pages = last - first + 1;
    int pps = (n_pages + p.splits_int2 - 1) / p.splits_int2;
    pps = (pps + 1) & ~1;
    const int p_begin = first + split * pps;
    const int p_end = min(min(first + n_pages, p_begin + pps), p.max_int2_pages);
    if (p_begin < p_end) {
      u32x4 bq[CT][3][2];
      const u32x4* qb = (const u32x4*)(p.qb + (int64_t)bk * CT * 3 * 2 * 64 * 4);
#pragma unroll
      for (int ct = 0; ct < CT; ++ct)
#pragma unroll
        for (int d = 0; d < 3; ++d)
#pragma unroll
          for (int ks = 0; ks < 2; ++ks) bq[ct][d][ks] = qb[((ct * 3 + d) * 2 + ks) * 64 + lane];
      const float pscale = exp2f(p.p_scale_exp);
      const int32_t* bt = p.int2_bt + (int64_t)b * p.max_int2_pages;
      const int64_t npg = p.n_int2_pages;
      for (int lp0 = p_begin; lp0 < p_end; lp0 += 2) {
        const bool has1 = lp0 + 1 < p_end;
        int pg0 = bt[lp0];
        int pg1 = has1 ? bt[lp0 + 1] : pg0;
        const bool ok0 = pg0 >= 0 && pg0 < npg;
        const bool ok1 = pg1 >= 0 && pg1 < npg;
        if (!ok0) pg0 = 0;
        if (!ok1) pg1 = pg0;
        const uint8_t* blk0 = block_ptr(p.int2_pages, pg0, p.n_kv, kv, L.bytes());
        const uint8_t* blk1 = block_ptr(p.int2_pages, pg1, p.n_kv, kv, L.bytes());
        const bool interior = has1 && ok0 && ok1 && lp0 * kPage >= lo && (lp0 + 2) * kPage <= hi;
        if (interior) {
          int2_pair<NG, CT, false>(p, blk0, blk1, lp0, p_end, lo, hi, bq, qbar2, qneg3, kfac, pscale, m_run, l_run, zsum,
                                   acc);
        } else {
          // pages with a bad id are masked out entirely
          const int lo_e = lo, hi_e = hi;
          const int pe = ok0 ? (ok1 ? p_end : lp0 + 1) : lp0;
          int2_pair<NG, CT, true>(p, blk0, blk1, lp0, pe, lo_e, hi_e, bq, qbar2, qneg3, kfac, pscale, m_run, l_run, zsum,
                                  acc);
        }
      }
    }
  }
  // ---- finalize: reduce per-lane partials, undo scales, write partials ----
  const int S = p.splits_int2 + p.splits_bf16;
  const float accscale = exp2f(23.f - p.p_scale_exp);  // MFMA sums p s (2c - 3) 2^(sp-24)
  constexpr int G = kHeadDim / NG;
#pragma unroll
  for (int ct = 0; ct < CT; ++ct) {
    const float l = sum_across_quads(l_run[ct]);
    const float z = sum_across_quads(zsum[ct]);
    // rows of this lane in the PV accumulator: (h, gamma) = 16ct + 4qd + r
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float zr = __shfl(z, 4 * qd + r);
      const int row = 16 * ct + 4 * qd + r;
      const int h = row / NG, gam_row = row % NG;
#pragma unroll
      for (int kt = 0; kt < 8; ++kt) {
        const int ch = 8 * ln + kt;
        if (h < p.g && ch / G == gam_row) {
          float* dst = p.partial + (((int64_t)b * p.n_q + kv * p.g + h) * S + split) * kPartialStride;
          dst[2 + ch] = fmaf(acc[ct][kt][r], accscale, zr);
        }
      }
    }
    const int col = 16 * ct + ln, h = col / NG;
    if (qd == 0 && col % NG == 0 && h < p.g) {
      float* dst = p.partial + (((int64_t)b * p.n_q + kv * p.g + h) * S + split) * kPartialStride;
      dst[0] = m_run[ct];
      dst[1] = l;
    }
  }
}

// ---------------------------------------------------------------------------
// main kernel: bf16 work item (sink + recent tokens, or the whole context in
// the all-bf16 baseline)
// ---------------------------------------------------------------------------
__device__ __forceinline__ bool bf16_slot_valid(int L, int n_sink, int ring0, int n_rec) {
  return L < n_sink || (L >= ring0 && L < ring0 + n_rec);
}

template <bool EDGE>
__device__ __forceinline__ void bf16_pair(const DecodeParams& p, const uint8_t* blk0, const uint8_t* blk1, int lp0,
                                          int p_end, int n_sink, int ring0, int n_rec, const u32x4 (&bq)[4],
                                          float& m_run, float& l_run, f32x4 (&acc)[8]) {
  const int lane = threadIdx.x, ln = lane & 15, qd = lane >> 4;
  const int a = qd & 1;
  const uint8_t* bk = (ln >> 3) ? blk1 : blk0;
  const int tokA = 8 * ((ln >> 2) & 1) + (ln & 3);
  u32x4 ka[2][4];
#pragma unroll
  for (int t = 0; t < 2; ++t)
#pragma unroll
    for (int s = 0; s < 4; ++s) ka[t][s] = *(const u32x4*)(bk + (tokA + 4 * t) * 256 + 64 * qd + 16 * s);
  const uint8_t* bq_ = (qd >> 1) ? blk1 : blk0;
  u32x4 vv[8];
#pragma unroll
  for (int kt = 0; kt < 8; ++kt) vv[kt] = *(const u32x4*)(bq_ + 4096 + ((8 * ln + kt) * 16 + 8 * a) * 2);

  f32x4 c[2];
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    c[t] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < 4; ++s) c[t] = mfma_bf16(ka[t][s], bq[s], c[t]);
  }
  const int lp = lp0 + (qd >> 1);
  bool valid[2][4];
  float lg[2][4];
  float mt = kNegInf;
#pragma unroll
  for (int t = 0; t < 2; ++t)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      if constexpr (EDGE) {
        const int L = lp * kPage + 8 * a + 4 * t + r;
        valid[t][r] = lp < p_end && bf16_slot_valid(L, n_sink, ring0, n_rec);
      } else {
        valid[t][r] = true;
      }
      lg[t][r] = valid[t][r] ? c[t][r] * kLog2eOverSqrtD : kNegInf;
      mt = fmaxf(mt, lg[t][r]);
    }
  mt = max_across_quads(mt);
  const float m_new = fmaxf(m_run, mt);
  if (__builtin_amdgcn_ballot_w64(m_new > m_run)) {
    const float alpha = (m_new == kNegInf) ? 1.f : exp2f(m_run - m_new);
    l_run *= alpha;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float ar = __shfl(alpha, 4 * qd + r);
#pragma unroll
      for (int kt = 0; kt < 8; ++kt) acc[kt][r] *= ar;
    }
    m_run = m_new;
  }
  float pr[2][4];
#pragma unroll
  for (int t = 0; t < 2; ++t)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float e = exp2f(lg[t][r] - m_run);
      pr[t][r] = valid[t][r] ? e : 0.f;
      l_run += pr[t][r];
    }
  // A register r: tokens 8a + 2r, 8a + 2r + 1 = tile r/2, rows 2(r%2), 2(r%2)+1.
  // p = hi + mid + lo in bf16 (24 significant bits): bf16 values are not
  // clipped, so a few large unrotated values can dominate the sum.
  u32x4 ph, pm, pl;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const float x0 = pr[r >> 1][2 * (r & 1)], x1 = pr[r >> 1][2 * (r & 1) + 1];
    const uint32_t h0 = bf16_bits(x0), h1 = bf16_bits(x1);
    const float r0 = x0 - bf16_val(h0), r1 = x1 - bf16_val(h1);
    const uint32_t m0 = bf16_bits(r0), m1 = bf16_bits(r1);
    ph[r] = h0 | (h1 << 16);
    pm[r] = m0 | (m1 << 16);
    pl[r] = bf16_bits(r0 - bf16_val(m0)) | (bf16_bits(r1 - bf16_val(m1)) << 16);
  }
#pragma unroll
  for (int kt = 0; kt < 8; ++kt) {
    acc[kt] = mfma_bf16(ph, vv[kt], acc[kt]);
    acc[kt] = mfma_bf16(pm, vv[kt], acc[kt]);
    acc[kt] = mfma_bf16(pl, vv[kt], acc[kt]);
  }
}

__device__ void bf16_item(const DecodeParams& p, int b, int kv, int split) {
  const int lane = threadIdx.x, ln = lane & 15, qd = lane >> 4;
  const int T = p.ctx_lens[b];
  const int n_sink = min(p.sink, T);
  const int ring0 = kPage * ((p.sink + kPage - 1) / kPage);
  const int n_rec = T > p.sink ? min(p.recent, T - p.sink) : 0;
  const int n_logical = (T <= p.sink) ? (T + kPage - 1) / kPage : ring0 / kPage + (n_rec + kPage - 1) / kPage;
  const int sb = split - p.splits_int2;
  float m_run = kNegInf, l_run = 0.f;
  f32x4 acc[8];
#pragma unroll
  for (int kt = 0; kt < 8; ++kt) acc[kt] = f32x4{0.f, 0.f, 0.f, 0.f};
  int pps = (n_logical + p.splits_bf16 - 1) / p.splits_bf16;
  pps = (pps + 1) & ~1;
  const int p_begin = sb * pps;
  const int p_end = min(min(n_logical, p_begin + pps), p.max_bf16_pages);
  if (p_begin < p_end) {
    u32x4 bq[4];
    const bool hv = ln < p.g;
    const uint16_t* qrow = p.q + ((int64_t)b * p.n_q + kv * p.g + (hv ? ln : 0)) * kHeadDim;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const u32x4 v = *(const u32x4*)(qrow + 32 * qd + 8 * s);
      bq[s] = hv ? v : u32x4{0u, 0u, 0u, 0u};
    }
    const int32_t* bt = p.bf16_bt + (int64_t)b * p.max_bf16_pages;
    const int64_t npg = p.n_bf16_pages;
    for (int lp0 = p_begin; lp0 < p_end; lp0 += 2) {
      const bool has1 = lp0 + 1 < p_end;
      int pg0 = bt[lp0];
      int pg1 = has1 ? bt[lp0 + 1] : pg0;
      const bool ok0 = pg0 >= 0 && pg0 < npg;
      const bool ok1 = pg1 >= 0 && pg1 < npg;
      if (!ok0) pg0 = 0;
      if (!ok1) pg1 = pg0;
      const uint8_t* blk0 = block_ptr(p.bf16_pages, pg0, p.n_kv, kv, kBf16BlockBytes);
      const uint8_t* blk1 = block_ptr(p.bf16_pages, pg1, p.n_kv, kv, kBf16BlockBytes);
      const int L0 = lp0 * kPage, L1 = (lp0 + 2) * kPage;
      const bool interior =
          has1 && ok0 && ok1 && ((L1 <= n_sink) || (L0 >= ring0 && L1 <= ring0 + n_rec));
      if (interior) {
        bf16_pair<false>(p, blk0, blk1, lp0, p_end, n_sink, ring0, n_rec, bq, m_run, l_run, acc);
      } else {
        const int pe = ok0 ? (ok1 ? p_end : lp0 + 1) : lp0;
        bf16_pair<true>(p, blk0, blk1, lp0, pe, n_sink, ring0, n_rec, bq, m_run, l_run, acc);
      }
    }
  }
  const int S = p.splits_int2 + p.splits_bf16;
  const float l = sum_across_quads(l_run);
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int h = 4 * qd + r;
    if (h < p.g) {
      float* dst = p.partial + (((int64_t)b * p.n_q + kv * p.g + h) * S + split) * kPartialStride;
#pragma unroll
      for (int kt = 0; kt < 8; ++kt) dst[2 + 8 * ln + kt] = acc[kt][r];
    }
  }
  if (qd == 0 && ln < p.g) {
    float* dst = p.partial + (((int64_t)b * p.n_q + kv * p.g + ln) * S + split) * kPartialStride;
    dst[0] = m_run;
    dst[1] = l;
  }
}

template <int NG, int CT>
__global__ __launch_bounds__(64) void decode_main(DecodeParams p) {
  const int S = p.splits_int2 + p.splits_bf16;
  const int item = blockIdx.x;
  const int split = item % S;
  const int bk = item / S;
  const int kv = bk % p.n_kv, b = bk / p.n_kv;
  if (split < p.splits_int2)
    int2_item<NG, CT>(p, b, kv, split);
  else
    bf16_item(p, b, kv, split);
}

// ---------------------------------------------------------------------------
// combine: LSE merge, R_V^T on the INT2 part, normalisation
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(128) void decode_combine(DecodeParams p) {
  const int bk = blockIdx.x;
  const int b = bk / p.n_kv, kv = bk % p.n_kv;
  const int j = threadIdx.x;
  const int S = p.splits_int2 + p.splits_bf16;
  __shared__ float ai[kHeadDim];
  const float* R = p.r_v + (int64_t)kv * kHeadDim * kHeadDim;
  for (int h = 0; h < p.g; ++h) {
    const int hq = kv * p.g + h;
    const float* base = p.partial + ((int64_t)b * p.n_q + hq) * S * kPartialStride;
    float M = kNegInf;
    for (int s = 0; s < S; ++s) M = fmaxf(M, base[s * kPartialStride]);
    float o = 0.f;
    float aint = 0.f, abf = 0.f, L = 0.f;
    if (M != kNegInf) {
      for (int s = 0; s < S; ++s) {
        const float ms = base[s * kPartialStride];
        const float w = (ms == kNegInf) ? 0.f : exp2f(ms - M);
        L = fmaf(w, base[s * kPartialStride + 1], L);
        const float v = w == 0.f ? 0.f : w * base[s * kPartialStride + 2 + j];
        if (s < p.splits_int2)
          aint += v;
        else
          abf += v;
      }
    }
    ai[j] = aint;
    __syncthreads();
    if (M != kNegInf) {
      float r = 0.f;
      if (p.splits_int2 > 0) {
        const float4* row = (const float4*)(R + j * kHeadDim);
#pragma unroll 8
        for (int i = 0; i < kHeadDim / 4; ++i) {
          const float4 rv = row[i];
          r = fmaf(ai[4 * i], rv.x, r);
          r = fmaf(ai[4 * i + 1], rv.y, r);
          r = fmaf(ai[4 * i + 2], rv.z, r);
          r = fmaf(ai[4 * i + 3], rv.w, r);
        }
      }
      o = (r + abf) / L;
    }
    p.out[((int64_t)b * p.n_q + hq) * kHeadDim + j] = o;
    __syncthreads();
  }
}

template <int NG, int CT>
hipError_t launch_decode_t(const DecodeParams& p, hipStream_t stream, hipEvent_t ev_start, hipEvent_t ev_stop) {
  const int bkn = p.batch * p.n_kv;
  const int S = p.splits_int2 + p.splits_bf16;
  if (p.splits_int2 > 0) {
    hipLaunchKernelGGL((decode_prologue<NG, CT>), dim3(bkn), dim3(128), 0, stream, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (ev_start) {
    hipError_t e = hipEventRecord(ev_start, stream);
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL((decode_main<NG, CT>), dim3(bkn * S), dim3(64), 0, stream, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (ev_stop) {
    e = hipEventRecord(ev_stop, stream);
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(decode_combine, dim3(bkn), dim3(128), 0, stream, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_decode(const DecodeParams& p, hipStream_t stream, hipEvent_t ev_start, hipEvent_t ev_stop) {
  if (p.ng == 4) {
    if (p.ct == 1) return launch_decode_t<4, 1>(p, stream, ev_start, ev_stop);
    if (p.ct == 2) return launch_decode_t<4, 2>(p, stream, ev_start, ev_stop);
    if (p.ct == 3) return launch_decode_t<4, 3>(p, stream, ev_start, ev_stop);
  } else if (p.ng == 2) {
    if (p.ct == 1) return launch_decode_t<2, 1>(p, stream, ev_start, ev_stop);
    if (p.ct == 2) return launch_decode_t<2, 2>(p, stream, ev_start, ev_stop);
    if (p.ct == 3) return launch_decode_t<2, 3>(p, stream, ev_start, ev_stop);
  }
  return hipErrorInvalidValue;
}

static size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

size_t decode_workspace_bytes(int batch, int n_q, int n_kv, int ct, int splits_total) {
  const size_t bkn = (size_t)batch * n_kv;
  return align256(bkn * ct * 3 * 2 * 64 * 4 * sizeof(uint32_t)) + align256(bkn * (1 + 32 * ct) * sizeof(float)) +
         align256((size_t)batch * n_q * splits_total * kPartialStride * sizeof(float));
}

void decode_workspace_carve(DecodeParams& p, void* ws) {
  const size_t bkn = (size_t)p.batch * p.n_kv;
  uint8_t* w = (uint8_t*)ws;
  p.qb = (uint32_t*)w;
  w += align256(bkn * p.ct * 3 * 2 * 64 * 4 * sizeof(uint32_t));
  p.qaux = (float*)w;
  w += align256(bkn * (1 + 32 * p.ct) * sizeof(float));
  p.partial = (float*)w;
}

}  // namespace oscar
