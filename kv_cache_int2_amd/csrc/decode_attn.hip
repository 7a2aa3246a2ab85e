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
//   decode_int2      per (request, KV head, split): one wavefront streams its
//                    share of INT2 pages, two pages (32 tokens) per iteration.
//   decode_bf16      the same for the bf16 pages (sink + recent tokens, or the
//                    whole context in the all-bf16 baseline).
//   decode_combine   per (request, KV head): log-sum-exp merge of the splits,
//                    R_V^T on the INT2 part, normalisation.
//
// INT2 logits on MFMA (int8, exact integer accumulation):
//   q~ = (q R_K) log2(e)/sqrt(d) is held as the fixed-point integer
//   Q = rint(q~ 2^sq) (|Q| <= 2^21 per (request, KV head)); 2Q is split into
//   three balanced int8 digits.  One MFMA per channel group gamma and four
//   heads (v_mfma_i32_16x16x32_i8 at G = 32, 16x16x64 at G = 64): K = the
//   group's channels, A = the digits, rows (head, digit), B = the 2-bit codes
//   as int8 bytes (columns = tokens).  Two shift-adds join a head's digit sums
//   into, exactly,
//     C = sum_{j in gamma} 2 Q_j c_j   (|C| < 2^29),   Qbar = sum_{j in gamma} Q_j,
//   and  sum_j 2 Q_j (z + c_j s) = s C + z 2 Qbar, two fp32 products whose
//   rounding (2^-24 of the larger term) stays far below the logit tolerance.
// INT2 values on MFMA (v_mfma_f32_16x16x32_f16):
//   A = P'[(h, gamma), t] = p_ht s_t,gamma 2^sp 4^-r as fp16 hi + lo (about 22
//   significant bits), B = the codes as exact fp16 subnormals c 4^r 2^-24 cut
//   from the packed bytes with one mask.  Odd token slots enter as -P' against
//   3 - c, so the products' signs alternate and the MFMA's accumulation stays
//   unbiased; the VALU sums p z and the 3 P' of the odd slots.  The
//   accumulator row (h, gamma) is kept for the channels of group gamma.
// bf16 tokens use v_mfma_f32_16x16x32_bf16 with the unrotated query (exact
// products) and P split into bf16 hi + mid + lo.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <cmath>
#include <mutex>
#include <type_traits>

#include "oscar_internal.h"
#include "quant_common.h"

namespace oscar {
namespace {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x1 __attribute__((ext_vector_type(1)));
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
__device__ __forceinline__ i32x4 mfma_i8_k32(u32x2 a, u32x2 b, i32x4 c) {
  return __builtin_amdgcn_mfma_i32_16x16x32_i8(__builtin_bit_cast(long, a), __builtin_bit_cast(long, b), c, 0, 0, 0);
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
// fp32 -> bf16 bits, nearest-even (finite inputs)
__device__ __forceinline__ uint32_t bf16_bits(float x) {
  uint32_t u = __builtin_bit_cast(uint32_t, x);
  return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}
__device__ __forceinline__ float bf16_val(uint32_t b) { return __builtin_bit_cast(float, b << 16); }
// x - (float)h for the low / high fp16 half of a packed pair, in one mixed-precision fma
__device__ __forceinline__ float mix_sub_lo(float x, f16x2 h) {
  float r;
  asm("v_fma_mix_f32 %0, -%1, 1.0, %2 op_sel_hi:[1,0,0]" : "=v"(r) : "v"(h), "v"(x));
  return r;
}
__device__ __forceinline__ float mix_sub_hi(float x, f16x2 h) {
  float r;
  asm("v_fma_mix_f32 %0, -%1, 1.0, %2 op_sel:[1,0,0] op_sel_hi:[1,0,0]" : "=v"(r) : "v"(h), "v"(x));
  return r;
}

// ((d0 << 8) + d1 << 8) + d2 as two shift-adds (v_lshl_add_u32): the empty asm
// keeps the compiler from re-associating it into two shifts and an add3.  The
// shift-adds stay compiler-generated, so the wait states after the MFMA that
// produced d0..d2 are the compiler's.
__device__ __forceinline__ int join_digits(int d0, int d1, int d2) {
  int t = (d0 << 8) + d1;
  asm("" : "+v"(t));
  return (t << 8) + d2;
}

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

// exp2 without the denormal-range fix-up: softmax weights below 2^-126 are 0
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// all-reduce max / sum over the 16 lanes of a row
__device__ __forceinline__ float row_max16(float x) {
  x = fmaxf(x, __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0xB1, 0xF, 0xF, false)));
  x = fmaxf(x, __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x4E, 0xF, 0xF, false)));
  x = fmaxf(x, __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x124, 0xF, 0xF, false)));
  x = fmaxf(x, __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x128, 0xF, 0xF, false)));
  return x;
}
__device__ __forceinline__ float row_sum16(float x) {
  x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0xB1, 0xF, 0xF, false));
  x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x4E, 0xF, 0xF, false));
  x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x124, 0xF, 0xF, false));
  x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x128, 0xF, 0xF, false));
  return x;
}

__device__ __forceinline__ const uint8_t* block_ptr(const uint8_t* base, int64_t page, int n_kv, int kv,
                                                    int bytes) {
  return base + ((page * n_kv + kv) * (int64_t)bytes);
}

// Element offset of the q (and out) row of kernel head hv of KV head kv, and
// the last position that head's query may attend (its own: the chunk's
// queries are the request's last positions; in decode, the last one).
__device__ __forceinline__ int64_t q_row(const DecodeParams& p, int b, int kv, int hv) {
  const int c = hv / p.g_real, h = hv - c * p.g_real;
  return (((int64_t)b * p.chunk + p.chunk0 + c) * p.q_heads + kv * p.g_real + h) * kHeadDim;
}
__device__ __forceinline__ int q_pos(const DecodeParams& p, int b, int hv) {
  return p.ctx_lens[b] - p.chunk + p.chunk0 + hv / p.g_real;
}

// Lane exchanges without LDS (a wavefront is four rows of 16 lanes): every
// lane takes the value n lanes around its row (DPP row rotate), or, from
// v_permlane16/32_swap with x in both registers, the values of the two rows it
// is paired with (rows (0,1) and (2,3); rows (0,2) and (1,3)).
// The swaps are written in asm: the compiler's builtins for them have handed
// back the first register for both results.  The s_nop 1 before gives the two
// wait states a swap needs after a VALU write of its operands; the one after
// gives the two a DPP read of a result needs (the compiler does not count an
// asm block as a VALU write).
template <bool ROWS32>
__device__ __forceinline__ void swap_rows(uint32_t& a, uint32_t& b) {
  if constexpr (ROWS32)
    asm volatile("s_nop 1\n\tv_permlane32_swap_b32 %0, %1\n\ts_nop 1" : "+v"(a), "+v"(b));
  else
    asm volatile("s_nop 1\n\tv_permlane16_swap_b32 %0, %1\n\ts_nop 1" : "+v"(a), "+v"(b));
}
__device__ __forceinline__ uint32_t lane_ror(uint32_t x, int n) {
  switch (n) {
    case 1: return (uint32_t)__builtin_amdgcn_mov_dpp((int)x, 0x121, 0xf, 0xf, false);
    case 2: return (uint32_t)__builtin_amdgcn_mov_dpp((int)x, 0x122, 0xf, 0xf, false);
    case 4: return (uint32_t)__builtin_amdgcn_mov_dpp((int)x, 0x124, 0xf, 0xf, false);
    default: return (uint32_t)__builtin_amdgcn_mov_dpp((int)x, 0x128, 0xf, 0xf, false);
  }
}
__device__ __forceinline__ double ror_f64(double v, int n) {
  const uint64_t u = __builtin_bit_cast(uint64_t, v);
  const uint64_t r = (uint64_t)lane_ror((uint32_t)u, n) | ((uint64_t)lane_ror((uint32_t)(u >> 32), n) << 32);
  return __builtin_bit_cast(double, r);
}
template <bool ROWS32>
__device__ __forceinline__ void row_pair_f64(double v, double& a, double& b) {
  const uint64_t u = __builtin_bit_cast(uint64_t, v);
  uint32_t l0 = (uint32_t)u, l1 = l0, h0 = (uint32_t)(u >> 32), h1 = h0;
  swap_rows<ROWS32>(l0, l1);
  swap_rows<ROWS32>(h0, h1);
  a = __builtin_bit_cast(double, (uint64_t)l0 | ((uint64_t)h0 << 32));
  b = __builtin_bit_cast(double, (uint64_t)l1 | ((uint64_t)h1 << 32));
}
// minimum and maximum of a double over the G (32 or 64) consecutive lanes of
// each group, in every lane: rows first (rotations by 1, 2, 4, 8), then row
// pairs.  Comparisons keep the current value against a NaN (a group holding
// NaN is flagged apart).
template <int G>
__device__ __forceinline__ void group_minmax_f64(double& mn, double& mx) {
#pragma unroll
  for (int n = 1; n < 16; n <<= 1) {
    const double a = ror_f64(mn, n), b = ror_f64(mx, n);
    mn = a < mn ? a : mn;
    mx = b > mx ? b : mx;
  }
  double a, b;
  row_pair_f64<false>(mn, a, b);
  mn = a < b ? a : b;
  row_pair_f64<false>(mx, a, b);
  mx = a > b ? a : b;
  if constexpr (G == 64) {
    row_pair_f64<true>(mn, a, b);
    mn = a < b ? a : b;
    row_pair_f64<true>(mx, a, b);
    mx = a > b ? a : b;
  }
}
// maximum of a non-negative float over the whole wavefront, in every lane
__device__ __forceinline__ float wave_max_nonneg(float x) {
  uint32_t u = __builtin_bit_cast(uint32_t, x);  // non-negative floats order as their bit patterns
#pragma unroll
  for (int n = 1; n < 16; n <<= 1) {
    const uint32_t y = lane_ror(u, n);
    u = y > u ? y : u;
  }
  uint32_t v = u;
  swap_rows<false>(u, v);
  u = v > u ? v : u;
  v = u;
  swap_rows<true>(u, v);
  u = v > u ? v : u;
  return __builtin_bit_cast(float, u);
}

// A 128 x 128 fp32 matrix to LDS by a block of 256 threads, row stride
// `stride` floats: 16 independent 16-byte loads per thread, all issued before
// the first store.
// t: this thread's index among the 256.
template <int Stride>
__device__ __forceinline__ void stage_matrix256(const float* src, float* lds, int t = threadIdx.x) {
  const float4* R = (const float4*)src;
  float4 v[16];
#pragma unroll
  for (int k = 0; k < 16; ++k) v[k] = R[t + 256 * k];
#pragma unroll
  for (int k = 0; k < 16; ++k) {
    const int e = t + 256 * k;
    float* d = lds + (e >> 5) * Stride + 4 * (e & 31);
    d[0] = v[k].x;
    d[1] = v[k].y;
    d[2] = v[k].z;
    d[3] = v[k].w;
  }
}

// ---------------------------------------------------------------------------
// decode-step writes, fused into the prologue
// ---------------------------------------------------------------------------
// Per (request, KV head), by the prologue's 256 threads: the token leaving the
// recent window is read from its bf16 slot and quantised into its INT2 slot; a
// new token that goes straight to the INT2 history is quantised from the
// input; a new sink/recent token is copied into its bf16 slot after the
// leaving token has been read (the two may share a ring slot).  The quantiser
// is the write path's: x R with exact bf16 x fp32 products summed in fp64,
// clip, per group mn/mx, s = fp16((mx - mn)/3), z = fp16(mn), code =
// clamp(rint((x - z)/s), 0, 3) in fp64, a group holding NaN stores NaN scale
// and zero with codes 0.  Thread t handles channel t % 128 of K (t < 128) or V.
struct StepScratch {
  float x[2][2][kHeadDim];     // [token][K/V][channel] inputs (bf16 values)
  uint8_t code[2][kHeadDim];   // [K/V][channel] codes of the token being stored
  uint32_t sz[2][4];           // [K/V][group] fp16 scale | zero << 16
};

template <int NG, int MB>
// wm: the matrix this work group writes (0 K, 1 V), -1 both; the threads of
// the other matrix (whole wavefronts) skip the arithmetic and the stores.
__device__ __forceinline__ void quantise_and_store(const DecodeParams& p, int kv, int tok, int32_t dst,
                                                   const float* rk, const float* rv, StepScratch& sc, int wm) {
  constexpr int G = kHeadDim / NG;
  constexpr Int2Layout L{NG, MB};
  const int t = threadIdx.x, m = t >> 7, j = t & (kHeadDim - 1);
  const bool mine = wm < 0 || m == wm;  // uniform per wavefront
  const float* R = m ? rv : rk;  // null: V arrives rotated (R_V folded into the V projection)
  const float* x = sc.x[tok][m];
  double acc = 0.0;
  if (mine) {
    if (R) {
#pragma unroll 8
      for (int i = 0; i < kHeadDim; i += 4) {
        const float4 x4 = *(const float4*)&x[i];
        acc = fma((double)x4.x, (double)R[i * kHeadDim + j], acc);
        acc = fma((double)x4.y, (double)R[(i + 1) * kHeadDim + j], acc);
        acc = fma((double)x4.z, (double)R[(i + 2) * kHeadDim + j], acc);
        acc = fma((double)x4.w, (double)R[(i + 3) * kHeadDim + j], acc);
      }
    } else {
      acc = (double)x[j];
    }
    const double tau = m ? p.tau_v : p.tau_k;
    const double v = acc < -tau ? -tau : (acc > tau ? tau : acc);
    double mn = v, mx = v;
    // the G channels of a group are consecutive lanes of one wavefront
    group_minmax_f64<G>(mn, mx);
    const uint64_t nan_lanes = __builtin_amdgcn_ballot_w64(v != v);
    const bool nan = G == 64 ? nan_lanes != 0 : ((nan_lanes >> (threadIdx.x & 32)) & 0xffffffffull) != 0;
    uint32_t pair = nan_sz<MB>();
    uint8_t c = 0;
    if (!nan) {
      double sd, zd;
      pair = encode_sz<MB>((mx - mn) / 3.0, mn, sd, zd);
      if (sd != 0.0) {
        double cd = __builtin_rint((v - zd) / sd);
        cd = cd < 0.0 ? 0.0 : (cd > 3.0 ? 3.0 : cd);
        c = (uint8_t)cd;
      }
    }
    sc.code[m][j] = c;
    if (j % G == 0) sc.sz[m][j / G] = pair;
  }
  __syncthreads();
  const int64_t page = dst / kPage;
  const int slot = dst % kPage;
  uint8_t* blk = p.int2_w + (page * p.n_kv + kv) * (int64_t)L.bytes();
  const bool do_k = wm != 1, do_v = wm != 0;
  if (do_k && t < 8) {
    // K codes, token-major: word t is word t%2 of quarter t/2; bits 2e hold
    // field e%4 of byte e/4
    uint32_t w = 0u;
#pragma unroll
    for (int e = 0; e < 16; ++e) w |= (uint32_t)sc.code[0][k_code_channel<NG>(t >> 1, t & 1, e >> 2, e & 3)] << (2 * e);
    *(uint32_t*)(blk + L.k_codes() + slot * 32 + 4 * t) = w;
  } else if (do_k && t >= 16 && t < 16 + NG) {
    const int gm = t - 16;
    store_sz<MB>(blk + L.k_sz() + (slot * NG + gm) * MB, sc.sz[0][gm]);  // K: token-major
  } else if (do_v && t >= 32 && t < 32 + NG) {
    const int gm = t - 32;
    store_sz<MB>(blk + L.v_sz() + (gm * kPage + slot) * MB, sc.sz[1][gm]);  // V: group-major
  } else if (do_v && t >= 64 && t < 96) {
    // V codes by token quad: byte jc of quad slot/4 holds channel jc, this
    // token at bits 2 (slot % 4); the other three tokens keep their bits
    const int jd = t - 64, sh = 2 * (slot & 3);
    uint32_t mask = 0u, bits = 0u;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      mask |= 3u << (8 * e + sh);
      bits |= (uint32_t)sc.code[1][4 * jd + e] << (8 * e + sh);
    }
    uint32_t* word = (uint32_t*)(blk + L.v_codes() + (slot >> 2) * kHeadDim + 4 * jd);
    atomicAnd(word, ~mask);
    atomicOr(word, bits);
  }
  __syncthreads();
}

// step slot row r (0-3) of request b: from the launch arguments or from the
// caller's device array
__device__ __forceinline__ int32_t step_slot(const DecodeParams& p, const ArgTables& tabs, int r, int b) {
  return p.arg_tables ? tabs.v[r][b] : p.step_slots[r * p.batch + b];
}

// wm: as for quantise_and_store (0 K, 1 V, -1 both)
template <int NG, int MB>
__device__ void step_writes(const DecodeParams& p, const ArgTables& tabs, int b, int kv, const float* rk,
                            const float* rv, StepScratch& sc, int wm) {
  const int t = threadIdx.x, m = t >> 7, j = t & (kHeadDim - 1);
  const bool mine = wm < 0 || m == wm;
  const int32_t i2_new = step_slot(p, tabs, 0, b), bf_new = step_slot(p, tabs, 1, b);
  const int32_t age_src = step_slot(p, tabs, 2, b), age_dst = step_slot(p, tabs, 3, b);
  const bool age = age_src >= 0 && age_dst >= 0 && age_src / kPage < p.n_bf16_pages &&
                   age_dst / kPage < p.n_int2_pages;
  const bool put_i2 = i2_new >= 0 && i2_new / kPage < p.n_int2_pages;
  const bool put_bf = bf_new >= 0 && bf_new / kPage < p.n_bf16_pages;
  const int64_t in = ((int64_t)b * p.n_kv + kv) * kHeadDim + j;
  const uint16_t xn = (m ? p.v_new : p.k_new)[in];
  // bf16 block: K [16][d] then V [d][16]
  auto bf16_elem = [&](int32_t slot_id) {
    uint16_t* blk = (uint16_t*)(p.bf16_w + ((int64_t)(slot_id / kPage) * p.n_kv + kv) * (int64_t)kBf16BlockBytes);
    const int sl = slot_id % kPage;
    return m ? blk + kPage * kHeadDim + j * kPage + sl : blk + sl * kHeadDim + j;
  };
  if (age && mine) sc.x[0][m][j] = bf16_val(*bf16_elem(age_src));
  if (put_i2 && mine) sc.x[1][m][j] = bf16_val(xn);
  __syncthreads();  // the leaving token has been read before its ring slot is reused
  if (put_bf && mine) *bf16_elem(bf_new) = xn;
  if (age) quantise_and_store<NG, MB>(p, kv, 0, age_dst, rk, rv, sc, wm);
  if (put_i2) quantise_and_store<NG, MB>(p, kv, 1, i2_new, rk, rv, sc, wm);
}

// The INT2 kernel's q operands of one (request, KV head), from the fixed-point
// q~ (qi: [head][channel], g heads) and its scale exponent sq, for `tiles`
// 16-row tiles (16/NG heads; heads past the g heads get zero digits):
// aux = [logit factor 2^-sq / 2, 2 Qbar per row], then the int8 digits of 2Q
// as MFMA A operands (digit 0 the most significant).  A tile of 16/NG heads
// takes four MFMAs per page, unit u = (head quad hq, group gam), u = hq NG +
// gam, each with K = the group's G channels and rows (head 4hq + ln/4 of the
// tile, digit ln%4; digit 3 is zero): words ((tile*4 + u)*64 + lane)*(8/NG) +
// reg, 8/NG registers per lane (16x16x32 MFMA at G = 32, 16x16x64 at G = 64).
// Byte i of reg j of lane quad a is channel G gam + (G/4) a + 4j + i: the key
// fields that (word >> 2m) & 0x03030303 delivers for that group.
// Called by all 256 threads after qi is complete.
template <int NG>
__device__ __forceinline__ void write_q_operands(const DecodeParams& p, int bk, int tiles, int g,
                                                 const int (*qi)[kHeadDim], int sq) {
  constexpr int G = kHeadDim / NG;
  const int t = threadIdx.x;
  float* aux = p.qaux + (int64_t)bk * (1 + 16 * tiles);
  if (t == 0) aux[0] = ldexpf(0.5f, -sq);
  // 2 Qbar per row (head, group): 16 threads per row, each summing G/16
  // channels, then a reduction over the 16 lanes
  for (int e = t; e < 16 * 16 * tiles; e += 256) {
    const int row = e >> 4, part = e & 15;
    const int h = row / NG, gam = row % NG;
    int sum = 0;
    if (h < g) {
#pragma unroll
      for (int c = 0; c < G / 16; ++c) sum += qi[h][gam * G + part * (G / 16) + c];
    }
#pragma unroll
    for (int off = 8; off >= 1; off >>= 1) sum += __shfl_xor(sum, off);
    if (part == 0) aux[1 + row] = 2.0f * (float)sum;
  }
  uint32_t* qb = p.qb + (int64_t)bk * tiles * 3 * 2 * 64 * 4;
  constexpr int kRegs = 8 / NG;
  for (int w = t; w < tiles * 4 * 64 * kRegs; w += 256) {
    const int j = w % kRegs, lane = (w / kRegs) & 63, u = (w / (kRegs * 64)) & 3, ct = w / (kRegs * 256);
    const int ln = lane & 15, qd = lane >> 4;
    const int hq = u / NG, gam = u % NG;
    const int h = (16 / NG) * ct + 4 * hq + (ln >> 2), digit = ln & 3;
    uint32_t word = 0;
    if (h < g && digit < 3) {
      for (int byte = 0; byte < 4; ++byte) {
        // balanced int8 digits of 2Q: 2Q = d0 2^16 + d1 2^8 + d2
        const int q = 2 * qi[h][G * gam + (G / 4) * qd + 4 * j + byte];
        const int d2 = ((q + 128) & 255) - 128;
        const int q1 = (q - d2) >> 8;
        const int d1 = ((q1 + 128) & 255) - 128;
        const int d0 = (q1 - d1) >> 8;
        const int dv = digit == 0 ? d0 : (digit == 1 ? d1 : d2);
        word |= (uint32_t)(dv & 0xff) << (8 * byte);
      }
    }
    qb[w] = word;
  }
}

// q~ partial sums of GM heads (the rows of qs; rows past the real heads hold
// zeros) for column j over the inputs [64 hf, 64 hf + 64): eight rows of R_K
// read at a time, every head in the same straight-line loop body
template <int GM>
__device__ __forceinline__ void qrk_partial(const float* rk, const float (*qs)[kHeadDim], int hf, int j,
                                            float (&acc)[GM]) {
#pragma unroll
  for (int h = 0; h < GM; ++h) acc[h] = 0.f;
  for (int i = 64 * hf; i < 64 * hf + 64; i += 8) {
    float r[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) r[u] = rk[(i + u) * kHeadDim + j];
#pragma unroll
    for (int h = 0; h < GM; ++h) {
      const float4 qa = *(const float4*)&qs[h][i], qb = *(const float4*)&qs[h][i + 4];
      float a = acc[h];
      a = fmaf(qa.x, r[0], a);
      a = fmaf(qa.y, r[1], a);
      a = fmaf(qa.z, r[2], a);
      a = fmaf(qa.w, r[3], a);
      a = fmaf(qb.x, r[4], a);
      a = fmaf(qb.y, r[5], a);
      a = fmaf(qb.z, r[6], a);
      a = fmaf(qb.w, r[7], a);
      acc[h] = a;
    }
  }
}

// the scale exponent sq that brings the largest |q~| (mx) to [2^20, 2^21),
// so that |2Q| <= 2^22 fits three balanced int8 digits
__device__ __forceinline__ int q_scale_exponent(float mx) {
  int sq = 0;
  if (mx > 0.f && mx < __builtin_huge_valf()) {
    int e;
    frexpf(mx, &e);          // mx in [2^(e-1), 2^e)
    sq = min(21 - e, 100);   // keeps the logit factor 2^-sq / 2 a normal float
  }
  return sq;
}

// ---------------------------------------------------------------------------
// prologue: q R_K operands
// ---------------------------------------------------------------------------
// Words per (request, KV head): A digits of 2Q (write_q_operands gives their
// order; 1536 words per row tile reserved), then aux floats [1 + 16*CT]: logit
// factor 2^-sq / 2, per row 2*Qbar (float).
// WRITE: the decode-step writes come first.  With p.split_writes = 1 the grid
// is twice B x Hkv: work groups [0, B Hkv) build the q operands and work
// groups [B Hkv, 2 B Hkv) do the step's writes, side by side (for small
// batches, where the doubled grid still runs in one round); with 2 it is
// three times B x Hkv, writer 2 bk + m doing matrix m (K, V) of pair bk and
// staging only its own R.
// tabs: the step tables of oscar_decode_step_host_tables (p.arg_tables); the
// q-operand block of (b, KV head 0) then copies b's context length to ctx_w,
// which the later kernels read as ctx_lens.
template <int NG, int MB, int CT, bool WRITE>
__global__ __launch_bounds__(256) void decode_prologue(DecodeParams p, ArgTables tabs) {
  const int nbk = p.batch * p.n_kv;
  const bool writer = WRITE && p.split_writes && (int)blockIdx.x >= nbk;
  const int wi = (int)blockIdx.x - nbk;
  const int bk = writer ? (p.split_writes == 2 ? wi >> 1 : wi) : (int)blockIdx.x;
  const int wm = writer && p.split_writes == 2 ? (wi & 1) : -1;  // the writer's matrix, -1: both
  const int b = bk / p.n_kv, kv = bk % p.n_kv;
  const int t = threadIdx.x, j = t & (kHeadDim - 1), hf = t >> 7;
  if (WRITE && p.arg_tables && !writer && kv == 0 && t == 0) p.ctx_w[b] = tabs.v[4][b];
  __shared__ float rk[kHeadDim * kHeadDim];
  __shared__ float qs[16][kHeadDim];
  __shared__ int qi[16][kHeadDim];
  __shared__ float red[4];
  __shared__ float rv[WRITE ? kHeadDim * kHeadDim : 1];
  __shared__ __attribute__((aligned(16))) StepScratch sc;
  const int g = p.g;
  if (WRITE && (!p.split_writes || writer)) {
    if (p.r_v && wm != 0) stage_matrix256<kHeadDim>(p.r_v + (int64_t)kv * kHeadDim * kHeadDim, rv);
    if (wm != 1) stage_matrix256<kHeadDim>(p.r_k + (int64_t)kv * kHeadDim * kHeadDim, rk);
    __syncthreads();
    step_writes<NG, MB>(p, tabs, b, kv, rk, p.r_v ? rv : nullptr, sc, wm);
    if (writer) return;  // uniform per work group
  } else {
    stage_matrix256<kHeadDim>(p.r_k + (int64_t)kv * kHeadDim * kHeadDim, rk);
  }
  // GM: the most heads a launch of this tile count has (g <= GM); rows g .. GM-1
  // of qs are zero, so every loop below runs over GM heads without a branch
  constexpr int GM = (16 * CT / NG) < 16 ? (16 * CT / NG) : 16;
  for (int e = t; e < GM * kHeadDim; e += 256)
    qs[e >> 7][e & (kHeadDim - 1)] =
        (e >> 7) < g ? bf16_val(p.q[q_row(p, b, kv, e >> 7) + (e & (kHeadDim - 1))]) : 0.f;
  __syncthreads();
  // q~[h][j]: this thread sums inputs i in [64 hf, 64 hf + 64) for every head;
  // the halves exchange partial sums through LDS and each thread keeps the
  // heads h = hf, hf + 2, ...
  float acc[GM];
  qrk_partial<GM>(rk, qs, hf, j, acc);
  __syncthreads();  // qs becomes the exchange: each half publishes the heads the other keeps
#pragma unroll
  for (int h = 0; h < GM; ++h)
    if ((h & 1) != hf) qs[h][j] = acc[h];
  __syncthreads();
  float qt[8];
  float mx = 0.f;
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const int h = hf + 2 * k;
    qt[k] = 0.f;
    if (2 * k < GM && h < g) {  // GM is even
      const float own = hf ? acc[2 * k + 1 < GM ? 2 * k + 1 : 0] : acc[2 * k];  // hf is uniform per wavefront
      qt[k] = (own + qs[h][j]) * kLog2eOverSqrtD;
      mx = fmaxf(mx, fabsf(qt[k]));
    }
  }

  mx = wave_max_nonneg(mx);
  if ((t & 63) == 0) red[t >> 6] = mx;
  __syncthreads();
  mx = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  const int sq = q_scale_exponent(mx);
#pragma unroll
  for (int k = 0; k < 8; ++k)
    if (hf + 2 * k < g) qi[hf + 2 * k][j] = (int)rintf(ldexpf(qt[k], sq));
  __syncthreads();
  write_q_operands<NG>(p, bk, CT, g, qi, sq);
}

// Prologue of a chunked-prefill launch: the same operands for up to 64 kernel
// heads (queries of the chunk x model heads of the KV head; the host keeps
// p.g <= 64), the heads taken 16 at a time; one scale exponent for all.
template <int NG>
__global__ __launch_bounds__(256) void prefill_prologue(DecodeParams p) {
  const int bk = blockIdx.x;
  const int b = bk / p.n_kv, kv = bk % p.n_kv;
  const int t = threadIdx.x, j = t & (kHeadDim - 1), hf = t >> 7;
  __shared__ float rk[kHeadDim * kHeadDim];
  __shared__ float qs[16][kHeadDim];
  __shared__ float qt[64][kHeadDim];
  __shared__ int qi[64][kHeadDim];
  __shared__ float red[4];
  const int g = p.g;
  stage_matrix256<kHeadDim>(p.r_k + (int64_t)kv * kHeadDim * kHeadDim, rk);
  float mx = 0.f;
  for (int h0 = 0; h0 < g; h0 += 16) {
    const int gb = min(16, g - h0);
    __syncthreads();  // R_K staged; the previous block's exchange is read
    for (int e = t; e < 16 * kHeadDim; e += 256)
      qs[e >> 7][e & (kHeadDim - 1)] =
          (e >> 7) < gb ? bf16_val(p.q[q_row(p, b, kv, h0 + (e >> 7)) + (e & (kHeadDim - 1))]) : 0.f;
    __syncthreads();
    float acc[16];
    qrk_partial<16>(rk, qs, hf, j, acc);
    __syncthreads();  // qs becomes the exchange of the halves' partial sums
#pragma unroll
    for (int h = 0; h < 16; ++h)
      if ((h & 1) != hf) qs[h][j] = acc[h];
    __syncthreads();
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const int h = hf + 2 * k;
      if (h < gb) {
        const float own = hf ? acc[2 * k + 1] : acc[2 * k];  // hf is uniform per wavefront
        const float v = (own + qs[h][j]) * kLog2eOverSqrtD;
        qt[h0 + h][j] = v;
        mx = fmaxf(mx, fabsf(v));
      }
    }
  }
  for (int off = 32; off >= 1; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off));
  if ((t & 63) == 0) red[t >> 6] = mx;
  __syncthreads();
  mx = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  const int sq = q_scale_exponent(mx);
  for (int e = t; e < g * kHeadDim; e += 256)
    qi[e >> 7][e & (kHeadDim - 1)] = (int)rintf(ldexpf(qt[e >> 7][e & (kHeadDim - 1)], sq));
  __syncthreads();
  write_q_operands<NG>(p, bk, p.ct, g, qi, sq);
}

// ---------------------------------------------------------------------------
// main kernel: INT2 work item
//
// Per iteration one wavefront takes two pages (32 tokens) of one (request, KV
// head).  Logits: C[(h, gamma), t] = sum_j 2Q_hj c_tj on the int8 MFMA with
// A = digits of 2Q (rows (h, gamma)), B = codes (columns = the 16 tokens of one
// page).  Lane l then holds, for the head of its row group and token l%16, all
// channel groups, so the group sum and the exp need no cross-lane traffic.
// The running max is lazy: it moves, with a margin, only when a logit passes
// it (one ballot per pair); only then are row maxima reduced and the
// accumulators rescaled.  p moves through LDS to the value MFMA, whose A
// operand is P'[(h, gamma), t] (rows again (h, gamma), k = tokens) and whose
// accumulator rows match the logit rows, so rescaling is lane-local.
//
// Value k order: in lane quad qd, half-word 2r + e of the operand is token
// 4qd + r of page e.  Both pages are then read at lane-uniform block
// addresses, and one byte permute pairs a channel's codes of the two pages.
// ---------------------------------------------------------------------------
constexpr float kMaxMargin = 4.f;  // log2 headroom added when the running max moves

template <int NG, int CT>
struct Int2State {
  static constexpr int HPL = 4 / NG;  // heads per lane per row tile
  // running max m (log2 units) kept as moff = log2(pfac) - m, so that the exp
  // yields p pfac directly; l sums those scaled weights (per lane)
  float moff[CT][HPL];
  float mx_run[CT][HPL];  // m in raw logit units
  float l_run[CT][HPL];
  // value-operand row 16ct + ln, units pscale 4^-r: zz[r] = sum over token slot
  // r of p z, plus 3 p s on the odd slots
  float zz[CT][4];
  f32x4 acc[CT][8];
};

template <int NG, int CT>
struct Int2Const {
  // digits of 2Q as A operands of unit u = (head quad u / NG, group u % NG),
  // rows (head, digit)
  typename std::conditional<NG == 4, u32x2, u32x4>::type qa[CT][4];
  float qbar2[CT][4];  // 2 Qbar of those rows
  float kfac, ikfac;   // raw logit -> log2 units, and its inverse (powers of two)
  float lpf;           // log2(pscale 4^-(ln % 4)): P' factor of the token this lane writes
};

// one pair of INT2 blocks, as this lane reads them: the key part, read
// before the logits, and the value part, read after the softmax
template <int NG>
struct Int2KData {
  u32x2 kc[2];          // K codes: token ln, bytes 8qd..8qd+7
  uint32_t ksz[2][NG];  // K (s, z): token ln, every group
};
template <int NG>
struct Int2VData {
  u32x2 vw[2];          // V codes: quad qd, channels 8ln..8ln+7
  u32x4 vsz[2];         // V (s, z): group ln % NG, tokens 4qd..4qd+3
};
// a pair already in registers (the masked path)
template <int NG>
struct Int2Data {
  Int2KData<NG> kd;
  Int2VData<NG> vd;
  __device__ __forceinline__ const Int2KData<NG>& k() const { return kd; }
  __device__ __forceinline__ const Int2VData<NG>& v() const { return vd; }
};

struct Int2Offsets {
  uint32_t kc, ksz, vw, vsz;
};

template <int NG, int MB>
__device__ __forceinline__ Int2Offsets int2_offsets() {
  constexpr Int2Layout L{NG, MB};
  const int lane = threadIdx.x & 63, ln = lane & 15, qd = lane >> 4;
  return Int2Offsets{(uint32_t)(L.k_codes() + ln * 32 + 8 * qd), (uint32_t)(L.k_sz() + ln * NG * MB),
                     (uint32_t)(L.v_codes() + qd * kHeadDim + 8 * ln),
                     (uint32_t)(L.v_sz() + ((ln % NG) * kPage + 4 * qd) * MB)};
}

// Stored (scale, zero) pairs -> fp16 pairs, scale in the low half (the form
// the arithmetic reads).  FP8 E4M3 byte pairs convert exactly: every E4M3
// value is an fp16 value.
__device__ __forceinline__ uint32_t e4m3_pair_lo(uint32_t w) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, false));
}
__device__ __forceinline__ uint32_t e4m3_pair_hi(uint32_t w) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, true));
}
// one token's K pairs, every group: NG stored pairs, raw words of 4 or 2 bytes each
template <int NG, int MB, class W>
__device__ __forceinline__ void k_pairs(const W& raw, uint32_t (&ksz)[NG]) {
#pragma unroll
  for (int g = 0; g < NG; ++g) {
    if constexpr (MB == 4)
      ksz[g] = raw[g];
    else
      ksz[g] = (g & 1) ? e4m3_pair_hi(raw[g >> 1]) : e4m3_pair_lo(raw[g >> 1]);
  }
}
// four tokens' V pairs of one group
template <int MB, class W>
__device__ __forceinline__ u32x4 v_pairs(const W& raw) {
  if constexpr (MB == 4)
    return raw;
  else
    return u32x4{e4m3_pair_lo(raw[0]), e4m3_pair_hi(raw[0]), e4m3_pair_lo(raw[1]), e4m3_pair_hi(raw[1])};
}
// raw words of a lane's K pairs (NG * MB bytes) and V pairs (4 * MB bytes)
template <int NG, int MB>
using KRaw = typename std::conditional<NG * MB == 16, u32x4, typename std::conditional<NG * MB == 8, u32x2, u32x1>::type>::type;
template <int MB>
using VRaw = typename std::conditional<MB == 4, u32x4, u32x2>::type;

// Buffer descriptor of one block (gfx9 raw buffer: stride 0, bounds = the
// block's bytes).  The block address is wavefront-uniform, so the descriptor
// lives in SGPRs and each load is a per-lane 32-bit offset with no address math.
constexpr int kBufferWord3 = 0x00020000;
// s_waitcnt immediate for vmcnt(0) alone (expcnt and lgkmcnt at their maxima)
constexpr int kWaitVmcnt0 = 0x0F70;

template <class W>
__device__ __forceinline__ W buffer_load(__amdgpu_buffer_rsrc_t rs, uint32_t off) {
  if constexpr (sizeof(W) == 16)
    return __builtin_amdgcn_raw_buffer_load_b128(rs, off, 0, 0);
  else if constexpr (sizeof(W) == 8)
    return __builtin_amdgcn_raw_buffer_load_b64(rs, off, 0, 0);
  else
    return u32x1{__builtin_amdgcn_raw_buffer_load_b32(rs, off, 0, 0)};
}

template <int NG, int MB>
__device__ __forceinline__ Int2Data<NG> int2_load(const uint8_t* blk0, const uint8_t* blk1, const Int2Offsets& o) {
  constexpr Int2Layout L{NG, MB};
  Int2Data<NG> d;
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const __amdgpu_buffer_rsrc_t rs =
        __builtin_amdgcn_make_buffer_rsrc((void*)(t ? blk1 : blk0), 0, L.bytes(), kBufferWord3);
    d.kd.kc[t] = __builtin_amdgcn_raw_buffer_load_b64(rs, o.kc, 0, 0);
    k_pairs<NG, MB>(buffer_load<KRaw<NG, MB>>(rs, o.ksz), d.kd.ksz[t]);
    d.vd.vw[t] = __builtin_amdgcn_raw_buffer_load_b64(rs, o.vw, 0, 0);
    d.vd.vsz[t] = v_pairs<MB>(buffer_load<VRaw<MB>>(rs, o.vsz));
  }
  return d;
}

// Interior pairs are staged through LDS with buffer->LDS loads (a pair is two
// blocks; each block is one full-wavefront 16-byte load plus one from the first
// (bytes - 1024)/16 lanes).  Such a load writes LDS at M0 + its immediate
// offset + 16 per lane, so the immediate stays 0 and the block offset travels
// in the per-lane offset.  The loads are issued from inline assembly: the
// compiler's wait insertion would otherwise put a full vmcnt(0) before every
// LDS read, which serialises the prefetch; vm_wait below carries the exact
// count instead (loads it does not know of can only lengthen its own waits).
// Ordering: the staging loads and the waits are compiler memory barriers, so
// no read of the staged bytes moves across them.  The loads carry the
// non-temporal hint: every history byte is read once per step, and streaming
// it past the caches' normal allocation measured about 13% more bandwidth.
__device__ __forceinline__ u32x4 block_rsrc(const void* p, uint32_t bytes) {
  const uint64_t a = (uint64_t)p;
  return u32x4{(uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)a),
               (uint32_t)__builtin_amdgcn_readfirstlane((int)((uint32_t)(a >> 32) & 0xffffu)), bytes,
               (uint32_t)kBufferWord3};
}
__device__ __forceinline__ uint32_t lds_address(const void* p) {
  return (uint32_t)(uintptr_t)(__attribute__((address_space(3))) const void*)p;
}
__device__ __forceinline__ void lds_dma16(const u32x4& rs, uint32_t lds, uint32_t voff) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, 0 offen nt lds"
               :
               : "s"(lds), "v"(voff), "s"(rs)
               : "memory", "m0");
}

// st: LDS byte address of a two-block slot
template <int NG, int MB>
__device__ __forceinline__ void int2_issue(const uint8_t* blk0, const uint8_t* blk1, uint32_t st) {
  constexpr Int2Layout L{NG, MB};
  constexpr int kRest = (L.bytes() - 1024) / 16;
  static_assert(L.bytes() > 1024 && L.bytes() <= 2048 && L.bytes() % 16 == 0, "block staging layout");
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const u32x4 rs = block_rsrc(t ? blk1 : blk0, L.bytes());
    lds_dma16(rs, st + t * L.bytes(), 16 * lane);
    if (lane < kRest) lds_dma16(rs, st + t * L.bytes() + 1024, 1024 + 16 * lane);
  }
}
// Wait until at most N vector-memory operations of this wavefront are in
// flight (the N most recent are the staging loads of the next one or two pairs).
template <int N>
__device__ __forceinline__ void vm_wait() {
  static_assert(N == 0 || N == 4 || N == 8, "vm_wait");
  if constexpr (N == 0)
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  else if constexpr (N == 4)
    asm volatile("s_waitcnt vmcnt(4)" ::: "memory");
  else
    asm volatile("s_waitcnt vmcnt(8)" ::: "memory");
}

// Workgroup barrier without a memory fence: a fence would make the staging
// wavefront drain the loads it keeps in flight.  The staged bytes a barrier
// publishes are complete by then (the staging wavefront's vm_wait comes
// first), and every wavefront has consumed the LDS data it read before it
// arrives; the "memory" clobber keeps LDS accesses on their side.
__device__ __forceinline__ void barrier_no_fence() { asm volatile("s_barrier" ::: "memory"); }

// a pair staged in LDS: each part is read when the pair asks for it
template <int NG, int MB>
struct Int2Staged {
  const uint8_t* st;
  Int2Offsets o;
  __device__ __forceinline__ Int2KData<NG> k() const {
    constexpr Int2Layout L{NG, MB};
    Int2KData<NG> d;
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const uint8_t* blk = st + t * L.bytes();
      d.kc[t] = *(const u32x2*)(blk + o.kc);
      k_pairs<NG, MB>(*(const KRaw<NG, MB>*)(blk + o.ksz), d.ksz[t]);
    }
    return d;
  }
  // wide tiles: (scale, zero) pairs of group gam, tokens 4qd .. 4qd + 3 of page t
  __device__ __forceinline__ u32x4 vsz_g(int t, int gam) const {
    constexpr Int2Layout L{NG, MB};
    const int qd = (threadIdx.x & 63) >> 4;
    return v_pairs<MB>(*(const VRaw<MB>*)(st + t * L.bytes() + L.v_sz() + (gam * kPage + 4 * qd) * MB));
  }
  // wide tiles: value B operand of channel tile T (channels 16T .. 16T + 15)
  __device__ __forceinline__ u32x4 v_wide(int T) const;
  __device__ __forceinline__ Int2VData<NG> v() const {
    constexpr Int2Layout L{NG, MB};
    Int2VData<NG> d;
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const uint8_t* blk = st + t * L.bytes();
      d.vw[t] = *(const u32x2*)(blk + o.vw);
      d.vsz[t] = v_pairs<MB>(*(const VRaw<MB>*)(blk + o.vsz));
    }
    return d;
  }
};

// MFMA B operands from packed codes.  Keys: one 32-bit word of 16 codes
// (4 per byte, at bits 2i) becomes the four int8 words of 4 codes each.
__device__ __forceinline__ u32x4 k_operand(uint32_t x) {
  return u32x4{x & 0x03030303u, (x >> 2) & 0x03030303u, (x >> 4) & 0x03030303u, (x >> 6) & 0x03030303u};
}
// Values, channel 8ln + kt: byte kt of this lane's quad, page 0 -> low half,
// page 1 -> high half; code c at bits 2r of each half is the fp16 subnormal
// c 2^(2r-24), and odd token slots take 3 - c = c ^ 3 (one and-xor)
__device__ __forceinline__ u32x4 v_operand(uint32_t lo_src, uint32_t hi_src, int kt) {
  const uint32_t sel = (uint32_t)(kt & 3) | 0x0c00u | ((uint32_t)(4 + (kt & 3)) << 16) | 0x0c000000u;
  const uint32_t x = __builtin_amdgcn_perm(hi_src, lo_src, sel);
  u32x4 bv;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const uint32_t m = 0x00030003u << (2 * r);
    bv[r] = (r & 1) ? ((x & m) ^ m) : (x & m);
  }
  return bv;
}
// Wide tiles (16 head rows, see int2_pair) take channel tiles of one group:
// tile T holds channels 16T + ln, one byte per page at quad qd.
template <int NG, int MB>
__device__ __forceinline__ u32x4 v_wide_operand(const uint8_t* st, int T) {
  constexpr Int2Layout L{NG, MB};
  const int lane = threadIdx.x & 63, ln = lane & 15, qd = lane >> 4;
  const int o = L.v_codes() + qd * kHeadDim + 16 * T + ln;
  return v_operand(st[o], st[L.bytes() + o], 0);
}
template <int NG, int MB>
__device__ __forceinline__ u32x4 Int2Staged<NG, MB>::v_wide(int T) const {
  return v_wide_operand<NG, MB>(st, T);
}

// EDGE: a masked pair.  Its tokens must lie in [lo, hi) on pages below
// p_end, and row head h (16 t0 ... of the wavefront's tiles) sees positions up
// to qlo + floor(h / g_real), i.e. position qlo + k when k g_real <= h (causal
// masks of a chunk's queries; in decode every row sees the whole INT2 region).
// LQ: head quads of the last tile that hold a real head (the others have zero
// digits: their logit MFMAs and sums are skipped, their logits taken as 0);
// 0 when the last tile has none.
// With one tile of 64-channel groups whose second head quad is empty, the
// value rows 8-15 (that quad's (head, group) rows) carry the lo part of rows
// 0-7 instead, so each channel tile takes one value MFMA, not two.
template <int NG, int CT, bool EDGE, int LQ, class Src>
__device__ __forceinline__ void int2_pair(const Src& src, int lp0, int p_end, int lo, int hi, int qlo, int g_real,
                                          int t0, const Int2Const<NG, CT>& K, Int2State<NG, CT>& S, float* p_lds) {
  constexpr int HPL = 4 / NG;
  constexpr bool kPackLo = NG == 2 && CT == 1 && LQ == 1;
  // wide: 16 heads per wavefront (four tiles at 32-channel groups, two at
  // 64); the value MFMAs take the 16 heads as rows against channel tiles of
  // one group each.  Head h is head h % 4 of quad entry (h / 4) % HPL of tile
  // h / (4 HPL).
  constexpr bool kWide = CT * HPL == 4;
  // one-tile bodies issue a page's logit MFMAs together, into accumulators of
  // their own (no MFMA-to-VALU wait after each); the two-tile bodies, held to
  // 168 VGPRs, and the wide ones join each unit's sums before the next MFMA
  constexpr bool kBatchUnits = CT == 1;
  const int lane = threadIdx.x & 63, ln = lane & 15, qd = lane >> 4;
  const int vrow = kPackLo ? (ln & 7) : ln;  // value-operand row this lane serves
  // ---- logits ----
  const Int2KData<NG> DK = src.k();
  bool seen[2][CT][HPL];
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const int pos = (lp0 + t) * kPage + ln;
    const bool valid = !EDGE || (lp0 + t < p_end && pos >= lo && pos < hi);
    const int later = __mul24(pos - qlo, g_real);  // |pos - qlo| < 2^17
#pragma unroll
    for (int ct = 0; ct < CT; ++ct)
#pragma unroll
      for (int hh = 0; hh < HPL; ++hh) {
        if constexpr (EDGE) {
          const int h = (16 / NG) * (t0 + ct) + 4 * hh + qd;
          seen[t][ct][hh] = valid && later <= h;
        } else {
          seen[t][ct][hh] = true;
        }
      }
  }
  float lg[2][CT][HPL];
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    u32x4 av[2];
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) av[ks] = k_operand(DK.kc[t][ks]);
#pragma unroll
    for (int ct = 0; ct < CT; ++ct) {
      // cd[u]: sum_j 2Q_j c_j of head 4hq + qd of the tile and group gam (u =
      // hq NG + gam), token ln: one MFMA per unit, whose rows (head, digit)
      // give this lane the three digit sums of that head.  Every partial
      // value is an exact integer below 2^31 in magnitude.
      auto unit_mfma = [&](int u) {
        const int gam = u % NG;
        if constexpr (NG == 4) {
          // group gam: fields 2(gam%2), +1 of word gam/2
          const u32x4& b4 = av[gam >> 1];
          const u32x2 bq = (gam & 1) ? u32x2{b4[2], b4[3]} : u32x2{b4[0], b4[1]};
          return mfma_i8_k32(K.qa[ct][u], bq, i32x4{0, 0, 0, 0});
        } else {
          return mfma_i8(K.qa[ct][u], av[gam], i32x4{0, 0, 0, 0});  // group gam: word gam
        }
      };
      auto skip = [&](int u) { return ct == CT - 1 && u / NG >= LQ; };
      i32x4 cd;
      if constexpr (kBatchUnits) {
        // the unit MFMAs issue together, into accumulators of their own, and
        // their digit sums are joined after them
        i32x4 ds[4];
#pragma unroll
        for (int u = 0; u < 4; ++u)
          if (!skip(u)) ds[u] = unit_mfma(u);
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          // at G = 64 the two-op join takes registers that body does not have
          const int c = NG == 4 ? join_digits(ds[u][0], ds[u][1], ds[u][2])
                                : (((ds[u][0] << 8) + ds[u][1]) << 8) + ds[u][2];
          cd[u] = skip(u) ? 0 : c;
        }
      } else {
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          if (skip(u)) {
            cd[u] = 0;
            continue;
          }
          const i32x4 d = unit_mfma(u);
          cd[u] = NG == 4 ? join_digits(d[0], d[1], d[2]) : (((d[0] << 8) + d[1]) << 8) + d[2];
        }
      }
#pragma unroll
      for (int hh = 0; hh < HPL; ++hh) {
        if (ct == CT - 1 && hh >= LQ) {
          lg[t][ct][hh] = seen[t][ct][hh] ? 0.f : kNegInf;
          continue;
        }
        float x = 0.f;
#pragma unroll
        for (int gg = 0; gg < NG; ++gg) {
          const int r = hh * NG + gg;
          const int c2 = cd[r];  // sum_j 2Q_j c_j
          const float sv = half_lo(DK.ksz[t][gg]), zv = half_hi(DK.ksz[t][gg]);
          x = fmaf(sv, (float)c2, fmaf(zv, K.qbar2[ct][r], x));
        }
        lg[t][ct][hh] = seen[t][ct][hh] ? x : kNegInf;
      }
    }
  }
  // ---- online softmax, lazy running max (per head: a 16-lane row) ----
  float pr[2][CT][HPL];
#pragma unroll
  for (int ct = 0; ct < CT; ++ct) {
    float mt[HPL];
    bool grow = false;
#pragma unroll
    for (int hh = 0; hh < HPL; ++hh) {
      mt[hh] = fmaxf(lg[0][ct][hh], lg[1][ct][hh]);
      grow |= mt[hh] > S.mx_run[ct][hh];
    }
    if (__builtin_expect(__builtin_amdgcn_ballot_w64(grow) != 0, 0)) {
      float alpha[HPL];
#pragma unroll
      for (int hh = 0; hh < HPL; ++hh) {
        const float rm = row_max16(mt[hh]);
        alpha[hh] = 1.f;
        if (rm > S.mx_run[ct][hh]) {
          const float m_new = fmaf(rm, K.kfac, kMaxMargin);
          const float moff = K.lpf - m_new;
          alpha[hh] = fast_exp2(moff - S.moff[ct][hh]);  // 0 when there was no max yet
          S.moff[ct][hh] = moff;
          S.mx_run[ct][hh] = m_new * K.ikfac;
          S.l_run[ct][hh] *= alpha[hh];
        }
      }
      // value-accumulator row 16ct + 4qd + r belongs to head (4qd + r) / NG of
      // the tile: at NG = 4 head qd, this lane's own; at NG = 2 head 2qd + r/2,
      // whose alpha quad (2qd + r/2) % 4 holds as entry (2qd + r/2) / 4
      if constexpr (kWide) {
        // accumulator row 4qd + e is head 4qd + e: tile qd / HPL, entry
        // qd % HPL, held by quad e; only the lanes of that tile's quads change
        const int ehh = HPL == 2 ? (qd & 1) : 0;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          float a = __shfl(alpha[0], 16 * e);
          if constexpr (HPL == 2) {
            const float a1 = __shfl(alpha[1], 16 * e);
            a = ehh ? a1 : a;
          }
#pragma unroll
          for (int kt = 0; kt < 8; ++kt) S.acc[0][kt][e] *= qd / HPL == ct ? a : 1.f;
        }
        // value row ln is head ln: tile ln / (4 HPL), entry (ln / 4) % HPL, quad ln % 4
        float az = __shfl(alpha[0], 16 * (ln & 3));
        if constexpr (HPL == 2) {
          const float az1 = __shfl(alpha[1], 16 * (ln & 3));
          az = ((ln >> 2) & 1) ? az1 : az;
        }
#pragma unroll
        for (int gam = 0; gam < NG; ++gam)
#pragma unroll
          for (int r = 0; r < 4; ++r) S.zz[gam][r] *= (ln >> 2) / HPL == ct ? az : 1.f;
      } else {
      float ar[2] = {alpha[0], alpha[0]};
      if constexpr (HPL == 2) {
#pragma unroll
        for (int e = 0; e < 2; ++e) {
          const int hl = 2 * (kPackLo ? (qd & 1) : qd) + e;
          const float x0 = __shfl(alpha[0], 16 * (hl & 3)), x1 = __shfl(alpha[1], 16 * (hl & 3));
          ar[e] = (hl >> 2) ? x1 : x0;
        }
      }
#pragma unroll
      for (int kt = 0; kt < 8; ++kt)
#pragma unroll
        for (int r = 0; r < 4; ++r) S.acc[ct][kt][r] *= ar[r >> 1];
      // value-operand row 16ct + ln belongs to head ln / NG of the tile, i.e.
      // 4hh + qd with qd = (ln / NG) % 4, hh = ln / (4 NG): its alpha is held
      // by quad qd, entry hh
      float az = __shfl(alpha[0], 16 * ((vrow / NG) & 3));
      if constexpr (HPL == 2) {
        const float az1 = __shfl(alpha[1], 16 * ((vrow / NG) & 3));
        az = (vrow >> 3) ? az1 : az;
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) S.zz[ct][r] *= az;
      }
    }
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int hh = 0; hh < HPL; ++hh) {
        const float e = fast_exp2(fmaf(lg[t][ct][hh], K.kfac, S.moff[ct][hh]));  // p pfac
        pr[t][ct][hh] = seen[t][ct][hh] ? e : 0.f;
        S.l_run[ct][hh] += pr[t][ct][hh];
      }
  }
  // ---- p' = p pscale 4^-(token % 4) to the value-operand layout: p_lds[h][page][16] ----
#pragma unroll
  for (int ct = 0; ct < CT; ++ct)
#pragma unroll
    for (int hh = 0; hh < HPL; ++hh) {
      const int h = (16 / NG) * ct + 4 * hh + qd;
#pragma unroll
      for (int t = 0; t < 2; ++t) p_lds[(2 * h + t) * kPage + ln] = pr[t][ct][hh];
    }
  __builtin_amdgcn_wave_barrier();
  if constexpr (kWide) {
    // ---- values, wide: A = P'[head ln][token] for one group at a time, B =
    // the group's channel tiles (8 / NG of 16 channels); rows are the 16 heads ----
    const f32x4 pf0 = *(const f32x4*)(p_lds + (2 * ln) * kPage + 4 * qd);
    const f32x4 pf1 = *(const f32x4*)(p_lds + (2 * ln + 1) * kPage + 4 * qd);
#pragma unroll
    for (int gam = 0; gam < NG; ++gam) {
      const u32x4 sz0 = src.vsz_g(0, gam), sz1 = src.vsz_g(1, gam);
      u32x4 ph, pl;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        float s0 = half_lo(sz0[r]), z0 = half_hi(sz0[r]);
        float s1 = half_lo(sz1[r]), z1 = half_hi(sz1[r]);
        if constexpr (EDGE) {
          // as below: a token without weight may hold a non-finite pair
          const bool v0 = pf0[r] != 0.f, v1 = pf1[r] != 0.f;
          s0 = v0 ? s0 : 0.f;
          z0 = v0 ? z0 : 0.f;
          s1 = v1 ? s1 : 0.f;
          z1 = v1 ? z1 : 0.f;
        }
        const float sg = (r & 1) ? -1.f : 1.f;
        const float x0 = fmaf(pf0[r], sg * s0, 0.f), x1 = fmaf(pf1[r], sg * s1, 0.f);
        const f16x2 hv = __builtin_bit_cast(f16x2, __builtin_amdgcn_cvt_pkrtz(x0, x1));
        ph[r] = __builtin_bit_cast(uint32_t, hv);
        pl[r] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(mix_sub_lo(x0, hv), mix_sub_hi(x1, hv)));
        S.zz[gam][r] = fmaf(pf0[r], z0, S.zz[gam][r]);
        S.zz[gam][r] = fmaf(pf1[r], z1, S.zz[gam][r]);
        if (r & 1) {
          S.zz[gam][r] = fmaf(-3.f, x0, S.zz[gam][r]);
          S.zz[gam][r] = fmaf(-3.f, x1, S.zz[gam][r]);
        }
      }
#pragma unroll
      for (int tt = 0; tt < 8 / NG; ++tt) {
        const int T = (8 / NG) * gam + tt;
        const u32x4 bv = src.v_wide(T);
        S.acc[0][T] = mfma_f16(ph, bv, S.acc[0][T]);
        S.acc[0][T] = mfma_f16(pl, bv, S.acc[0][T]);
      }
    }
    return;
  }
  const Int2VData<NG> DV = src.v();
  u32x4 pa[CT][2];
#pragma unroll
  for (int ct = 0; ct < CT; ++ct) {
    const int h = (16 * ct + vrow) / NG;
    const f32x4 pf0 = *(const f32x4*)(p_lds + (2 * h) * kPage + 4 * qd);
    const f32x4 pf1 = *(const f32x4*)(p_lds + (2 * h + 1) * kPage + 4 * qd);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      float s0 = half_lo(DV.vsz[0][r]), z0 = half_hi(DV.vsz[0][r]);
      float s1 = half_lo(DV.vsz[1][r]), z1 = half_hi(DV.vsz[1][r]);
      if constexpr (EDGE) {
        // a token this row gives no weight (an unwritten slot, a position its
        // query does not see) may hold a non-finite pair, and 0 * NaN is NaN:
        // zero its scale and zero point
        const bool v0 = pf0[r] != 0.f, v1 = pf1[r] != 0.f;
        s0 = v0 ? s0 : 0.f;
        z0 = v0 ? z0 : 0.f;
        s1 = v1 ? s1 : 0.f;
        z1 = v1 ? z1 : 0.f;
      }
      // odd token slots enter with -P' against the complemented code 3 - c
      const float sg = (r & 1) ? -1.f : 1.f;
      const float x0 = fmaf(pf0[r], sg * s0, 0.f), x1 = fmaf(pf1[r], sg * s1, 0.f);
      // hi = x truncated to fp16, lo = the exact remainder, truncated again
      const f16x2 hv = __builtin_bit_cast(f16x2, __builtin_amdgcn_cvt_pkrtz(x0, x1));
      const uint32_t lov = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(mix_sub_lo(x0, hv), mix_sub_hi(x1, hv)));
      if constexpr (kPackLo) {
        pa[ct][0][r] = ln < 8 ? __builtin_bit_cast(uint32_t, hv) : lov;
      } else {
        pa[ct][0][r] = __builtin_bit_cast(uint32_t, hv);
        pa[ct][1][r] = lov;
      }
      S.zz[ct][r] = fmaf(pf0[r], z0, S.zz[ct][r]);
      S.zz[ct][r] = fmaf(pf1[r], z1, S.zz[ct][r]);
      if (r & 1) {  // x = -p s pscale 4^-r here
        S.zz[ct][r] = fmaf(-3.f, x0, S.zz[ct][r]);
        S.zz[ct][r] = fmaf(-3.f, x1, S.zz[ct][r]);
      }
    }
  }
  // ---- values on MFMA ----
#pragma unroll
  for (int kt = 0; kt < 8; ++kt) {
    const u32x4 bv = v_operand(DV.vw[0][kt >> 2], DV.vw[1][kt >> 2], kt);
#pragma unroll
    for (int ct = 0; ct < CT; ++ct) {
      S.acc[ct][kt] = mfma_f16(pa[ct][0], bv, S.acc[ct][kt]);
      if constexpr (!kPackLo) S.acc[ct][kt] = mfma_f16(pa[ct][1], bv, S.acc[ct][kt]);
    }
  }
}

// W wavefronts per work item: wavefront w takes the CT row tiles starting at
// tile w CT, all of them reading the same staged pages; LQ as for int2_pair.
// edge_lds: this wavefront's two-block area for masked pairs (wide tiles only).
template <int NG, int MB, int CT, int W, int LQ>
__device__ void int2_item(const DecodeParams& p, int b, int kv, int split, float* p_lds, uint8_t* stage,
                          uint8_t* edge_lds) {
  constexpr Int2Layout L{NG, MB};
  constexpr int HPL = 4 / NG;
  constexpr int kTiles = W * CT;  // row tiles of the (request, KV head)
  constexpr bool kPackLo = NG == 2 && CT == 1 && LQ == 1;  // as in int2_pair
  constexpr bool kWide = CT * HPL == 4;                    // as in int2_pair
  const int lane = threadIdx.x & 63, ln = lane & 15, qd = lane >> 4;
  // first row tile of this wavefront (wavefront-uniform: kept in a scalar register)
  const int t0 = W > 1 ? __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6)) * CT : 0;
  const int T = p.ctx_lens[b];
  // the launch's queries sit at positions qlo .. qlo + (g - 1) / g_real (in
  // decode, T - 1 alone): keys up to qlo are seen by every row, later ones
  // (a chunk longer than the recent window) only by the rows of later queries
  const int qlo = T - p.chunk + p.chunk0;
  const int lo = p.sink;
  const int hi = min(T - p.recent, qlo + (p.g - 1) / p.g_real + 1);
  const int hi_all = min(hi, qlo + 1);
  const int g_real = p.g_real;
  const int bk = b * p.n_kv + kv;
  Int2State<NG, CT> S;
#pragma unroll
  for (int ct = 0; ct < CT; ++ct) {
#pragma unroll
    for (int hh = 0; hh < HPL; ++hh) {
      S.moff[ct][hh] = __builtin_huge_valf();
      S.mx_run[ct][hh] = kNegInf;
      S.l_run[ct][hh] = 0.f;
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) S.zz[ct][r] = 0.f;
#pragma unroll
    for (int kt = 0; kt < 8; ++kt) S.acc[ct][kt] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  const float* aux = p.qaux + (int64_t)bk * (1 + 16 * kTiles);
  const float pscale = exp2f(p.p_scale_exp);
  if (hi > lo && lo >= 0) {
    const int first = lo / kPage, last = (hi - 1) / kPage;
    const int n_pages = last - first + 1;
    int pps = (n_pages + p.splits_int2 - 1) / p.splits_int2;
    pps = (pps + 1) & ~1;
    const int p_begin = first + split * pps;
    const int p_end = min(min(first + n_pages, p_begin + pps), p.max_int2_pages);
    if (p_begin < p_end) {
      Int2Const<NG, CT> K;
      const uint32_t* qb = p.qb + (int64_t)bk * kTiles * 3 * 2 * 64 * 4;
#pragma unroll
      for (int ct = 0; ct < CT; ++ct) {
        using QA = typename std::conditional<NG == 4, u32x2, u32x4>::type;
#pragma unroll
        for (int u = 0; u < 4; ++u) K.qa[ct][u] = ((const QA*)qb)[((t0 + ct) * 4 + u) * 64 + lane];
        // 2 Qbar of (head 4hh + qd of the tile, group gg), r = hh NG + gg
#pragma unroll
        for (int r = 0; r < 4; ++r)
          K.qbar2[ct][r] = aux[1 + 16 * (t0 + ct) + NG * (4 * (r / NG) + qd) + r % NG];
      }
      K.kfac = aux[0];
      K.ikfac = 1.0f / K.kfac;
      K.lpf = p.p_scale_exp - (float)(2 * (ln & 3));
      const int32_t* bt = p.int2_bt + (int64_t)b * p.max_int2_pages;
      const int64_t npg = p.n_int2_pages;
      const uint8_t* base = p.int2_pages;
      const int n_kv = p.n_kv;
      const Int2Offsets off = int2_offsets<NG, MB>();
      auto blk = [&](int pg) { return base + ((int64_t)pg * n_kv + kv) * (int64_t)L.bytes(); };
      auto ok = [&](int pg) { return pg >= 0 && pg < npg; };
      // masked pair: partial pages at the region edges, odd tails, bad page ids
      auto edge = [&](int lp0) {
        const bool has1 = lp0 + 1 < p_end;
        int pg0 = bt[lp0];
        int pg1 = has1 ? bt[lp0 + 1] : pg0;
        const bool ok0 = ok(pg0), ok1 = ok(pg1);
        if (!ok0) pg0 = 0;
        if (!ok1) pg1 = pg0;
        const int pe = ok0 ? (ok1 ? p_end : lp0 + 1) : lp0;
        if constexpr (kWide) {
          // wide tiles read their operands from LDS: the two blocks are copied
          // into this wavefront's own area (16 bytes per lane and load; the
          // wavefront's LDS accesses complete in order)
          constexpr int n16 = L.bytes() / 16;
#pragma unroll
          for (int t = 0; t < 2; ++t) {
            const uint4* src = (const uint4*)blk(t ? pg1 : pg0);
            uint4* dst = (uint4*)(edge_lds + t * L.bytes());
            for (int c = lane; c < n16; c += 64) dst[c] = src[c];
          }
          int2_pair<NG, CT, true, LQ>(Int2Staged<NG, MB>{edge_lds, off}, lp0, pe, lo, hi, qlo, g_real, t0, K,
                                             S, p_lds);
        } else {
          const Int2Data<NG> D = int2_load<NG, MB>(blk(pg0), blk(pg1), off);
          int2_pair<NG, CT, true, LQ>(D, lp0, pe, lo, hi, qlo, g_real, t0, K, S, p_lds);
        }
      };
      int lp0 = p_begin;
      if (lp0 * kPage < lo) {
        edge(lp0);
        lp0 += 2;
      }
      // interior pairs (both pages fully inside [lo, hi_all)), staged in LDS two
      // pairs ahead in a ring of three slots.  Page ids come 64 at a time, one
      // per lane, and a pair takes its two ids with v_readlane: no memory
      // access and no wait inside the pair loop.  Each chunk ends with its
      // staging loads drained.
      const int main_end = min(p_end, hi_all / kPage);
      constexpr int kSlot = 2 * L.bytes();
      const uint32_t a0 = lds_address(stage);
      if constexpr (W == 1) {
        while (lp0 + 2 <= main_end) {
          const int c0 = lp0;
          const int cn = min(64, main_end - c0);
          const int id = lane < cn ? bt[c0 + lane] : 0;
          const uint64_t bad = __builtin_amdgcn_ballot_w64(lane < cn && !ok(id));
          const int lim = bad ? c0 + (int)__builtin_ctzll(bad) : c0 + cn;  // pages [c0, lim) have good ids
          if (lp0 + 2 > lim) break;
          // every earlier vector load (operands, ids, edge pages) completes here,
          // where the compiler sees it, so it adds no wait inside the pair loop
          __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
          auto page = [&](int l) { return blk(__builtin_amdgcn_readlane(id, l - c0)); };
          int2_issue<NG, MB>(page(lp0), page(lp0 + 1), a0);
          if (lp0 + 4 <= lim) int2_issue<NG, MB>(page(lp0 + 2), page(lp0 + 3), a0 + kSlot);
          int cur = 0;  // slot of the pair at lp0 (wavefront-uniform)
          for (;;) {
            // stage the pair two ahead into the slot the previous pair freed,
            // then wait for this pair's bytes
            const int nxt = cur == 0 ? 2 : cur - 1;
            if (lp0 + 6 <= lim) {
              int2_issue<NG, MB>(page(lp0 + 4), page(lp0 + 5), a0 + nxt * kSlot);
              vm_wait<8>();
            } else if (lp0 + 4 <= lim) {
              vm_wait<4>();
            } else {
              vm_wait<0>();
            }
            int2_pair<NG, CT, false, LQ>(Int2Staged<NG, MB>{stage + cur * kSlot, off}, lp0, p_end, lo, hi, qlo,
                                            g_real, t0, K, S, p_lds);
            lp0 += 2;
            if (lp0 + 2 > lim) break;
            cur = cur == 2 ? 0 : cur + 1;
          }
          if (lim < c0 + cn) break;  // a bad id: the rest goes through the masked path
        }
      } else {
        // the W wavefronts share one ring of four slots: wavefront 0 stages
        // two pairs ahead and waits for its loads; one barrier per pair then
        // publishes the pair to all and certifies that all have finished the
        // pair before last, whose slot the next staging load reuses
        const bool leader = t0 == 0;
        // (each wavefront unpacks its own code operands: sharing them through
        // LDS took a second barrier per pair, which cost more than it saved
        // for 3, 4 wide and 8 one-tile wavefronts)
        while (lp0 + 2 <= main_end) {
          const int c0 = lp0;
          const int cn = min(64, main_end - c0);
          const int id = lane < cn ? bt[c0 + lane] : 0;
          const uint64_t bad = __builtin_amdgcn_ballot_w64(lane < cn && !ok(id));
          const int lim = bad ? c0 + (int)__builtin_ctzll(bad) : c0 + cn;
          if (lp0 + 2 > lim) break;
          __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
          barrier_no_fence();  // every wavefront is done with the slots of the previous chunk
          auto page = [&](int l) { return blk(__builtin_amdgcn_readlane(id, l - c0)); };
          if (leader) {
            int2_issue<NG, MB>(page(lp0), page(lp0 + 1), a0);
            if (lp0 + 4 <= lim) int2_issue<NG, MB>(page(lp0 + 2), page(lp0 + 3), a0 + kSlot);
          }
          int cur = 0;
          for (;;) {
            if (leader) {
              if (lp0 + 6 <= lim) {
                int2_issue<NG, MB>(page(lp0 + 4), page(lp0 + 5), a0 + ((cur + 2) & 3) * kSlot);
                vm_wait<8>();
              } else if (lp0 + 4 <= lim) {
                vm_wait<4>();
              } else {
                vm_wait<0>();
              }
            }
            barrier_no_fence();
            int2_pair<NG, CT, false, LQ>(Int2Staged<NG, MB>{stage + cur * kSlot, off}, lp0, p_end, lo, hi, qlo,
                                                g_real, t0, K, S, p_lds);
            lp0 += 2;
            if (lp0 + 2 > lim) break;
            cur = (cur + 1) & 3;
          }
          if (lim < c0 + cn) break;
        }
      }
      for (; lp0 < p_end; lp0 += 2) edge(lp0);
    }
  }
  // ---- finalize ----
  const int Ssp = p.splits_int2 + p.splits_bf16;
  // the MFMA sums 2^(sp-24) (sum_even p s c - sum_odd p s (3 - c))
  const float accscale = exp2f(24.f - p.p_scale_exp);
  const float ipscale = 1.0f / pscale;
  constexpr int G = kHeadDim / NG;
  if constexpr (kWide) {
    // accumulator T, row 4qd + e: head 4 HPL t0 + 4qd + e, channel 16T + ln
    // (group T / (8 / NG)); the zero-point sums of value row (head) ln, group
    // gam, summed over the quads
    float zg[NG];
#pragma unroll
    for (int gam = 0; gam < NG; ++gam) {
      float z = 0.f;
#pragma unroll
      for (int r = 0; r < 4; ++r) z = fmaf(S.zz[gam][r], (float)(1 << (2 * r)) * ipscale, z);
      zg[gam] = sum_across_quads(z);
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int h = 4 * HPL * t0 + 4 * qd + e;
      float* dst = p.partial + (((int64_t)b * p.n_q + kv * p.g + h) * Ssp + split) * kPartialStride;
#pragma unroll
      for (int T = 0; T < 8; ++T) {
        const float zr = __shfl(zg[T / (8 / NG)], 4 * qd + e);
        if (h < p.g) dst[2 + 16 * T + ln] = fmaf(S.acc[0][T][e], accscale, zr);
      }
    }
  }
#pragma unroll
  for (int ct = 0; ct < CT; ++ct) {
    if constexpr (!kWide) {
    // sum p z + 3 sum_odd p s
    float z = 0.f;
#pragma unroll
    for (int r = 0; r < 4; ++r) z = fmaf(S.zz[ct][r], (float)(1 << (2 * r)) * ipscale, z);
    z = sum_across_quads(z);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float zr = __shfl(z, 4 * qd + r);
      const int row = 16 * (t0 + ct) + 4 * qd + r;
      const int h = row / NG, gam_row = row % NG;
#pragma unroll
      for (int kt = 0; kt < 8; ++kt) {
        const int ch = 8 * ln + kt;
        float a = S.acc[ct][kt][r];
        // packed lo rows: row 8 + i (lane quads 2, 3) adds onto row i (a
        // head of the empty quad is >= g, so quads 2, 3 store nothing)
        if constexpr (kPackLo) a += __shfl(a, lane + 32);
        if (h < p.g && ch / G == gam_row) {
          float* dst = p.partial + (((int64_t)b * p.n_q + kv * p.g + h) * Ssp + split) * kPartialStride;
          dst[2 + ch] = fmaf(a, accscale, zr);
        }
      }
    }
    }
#pragma unroll
    for (int hh = 0; hh < HPL; ++hh) {
      const float lpf = p.p_scale_exp - (float)(2 * (ln & 3));
      const float l = row_sum16(S.l_run[ct][hh] * exp2f(-lpf));
      const int h = (16 / NG) * (t0 + ct) + 4 * hh + qd;
      if (ln == 0 && h < p.g) {
        float* dst = p.partial + (((int64_t)b * p.n_q + kv * p.g + h) * Ssp + split) * kPartialStride;
        dst[0] = lpf - S.moff[ct][hh];  // -inf when this split saw no token
        dst[1] = l;
      }
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
// position held by a valid bf16 logical slot of a request of T positions: a
// sink slot holds its own position, ring slot r the newest position p < T
// with p - sink = r modulo the window
__device__ __forceinline__ int bf16_slot_position(int L, int ring0, int T, int sink, int window) {
  if (L < ring0) return L;
  const int r = L - ring0;
  return T - 1 - (T - 1 - sink - r) % window;
}

// EDGE: masked pair; its slots must be valid and hold positions <= qpos
// a pair of bf16 blocks as this lane reads them: K as the logits' A operand
// (tokens 8 ((ln / 4) % 2) + ln % 4 + 4t of page ln / 8), V as the values' B
// operand (channel 8 ln + kt, tokens 8 (qd % 2) .. + 7 of page qd / 2)
struct Bf16PairData {
  u32x4 ka[2][4];
  u32x4 vv[8];
};
__device__ __forceinline__ Bf16PairData bf16_pair_load(const uint8_t* blk0, const uint8_t* blk1) {
  const int lane = threadIdx.x & 63, ln = lane & 15, qd = lane >> 4;
  const int a = qd & 1;
  const uint8_t* bk = (ln >> 3) ? blk1 : blk0;
  const int tokA = 8 * ((ln >> 2) & 1) + (ln & 3);
  Bf16PairData d;
#pragma unroll
  for (int t = 0; t < 2; ++t)
#pragma unroll
    for (int s = 0; s < 4; ++s) d.ka[t][s] = *(const u32x4*)(bk + (tokA + 4 * t) * 256 + 64 * qd + 16 * s);
  const uint8_t* bq_ = (qd >> 1) ? blk1 : blk0;
#pragma unroll
  for (int kt = 0; kt < 8; ++kt) d.vv[kt] = *(const u32x4*)(bq_ + 4096 + ((8 * ln + kt) * 16 + 8 * a) * 2);
  return d;
}

template <bool EDGE>
__device__ __forceinline__ void bf16_pair(const DecodeParams& p, const Bf16PairData& d, int lp0, int p_end,
                                          int n_sink, int ring0, int n_rec, int T, int qpos, const u32x4 (&bq)[4],
                                          float& m_run, float& l_run, f32x4 (&acc)[8]) {
  const int lane = threadIdx.x & 63, qd = lane >> 4;
  const int a = qd & 1;
  const u32x4 (&ka)[2][4] = d.ka;
  u32x4 vv[8];
#pragma unroll
  for (int kt = 0; kt < 8; ++kt) vv[kt] = d.vv[kt];

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
        valid[t][r] = lp < p_end && bf16_slot_valid(L, n_sink, ring0, n_rec) &&
                      bf16_slot_position(L, ring0, T, p.sink, p.recent) <= qpos;
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
  if constexpr (EDGE) {
    // a masked slot may hold a non-finite value (an unwritten slot, a
    // position the query does not see): zero it, since 0 * NaN is NaN.
    // Value word w of this lane holds its tokens 8a + 2w and 8a + 2w + 1.
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const uint32_t keep = (valid[w >> 1][2 * (w & 1)] ? 0x0000ffffu : 0u) |
                            (valid[w >> 1][2 * (w & 1) + 1] ? 0xffff0000u : 0u);
#pragma unroll
      for (int kt = 0; kt < 8; ++kt) vv[kt][w] &= keep;
    }
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

// The bf16 region of one (request, KV head) for query c of the launch (its
// g_real model heads, rows ln < g_real), split `split` of the partials.
// PREFETCH: the next pair's blocks are read before the current pair is
// computed (for the combine kernel, whose wavefronts have registers to spare).
template <bool PREFETCH>
__device__ void bf16_item(const DecodeParams& p, int b, int kv, int split, int c) {
  const int lane = threadIdx.x & 63, ln = lane & 15, qd = lane >> 4;
  const int T = p.ctx_lens[b];
  const int h0 = c * p.g_real;  // first kernel head of this query
  const int qpos = q_pos(p, b, h0);
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
    const bool hv = ln < p.g_real;
    const uint16_t* qrow = p.q + q_row(p, b, kv, h0 + (hv ? ln : 0));
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const u32x4 v = *(const u32x4*)(qrow + 32 * qd + 8 * s);
      bq[s] = hv ? v : u32x4{0u, 0u, 0u, 0u};
    }
    const int32_t* bt = p.bf16_bt + (int64_t)b * p.max_bf16_pages;
    const int64_t npg = p.n_bf16_pages;
    // the split's page ids, 64 at a time, one per lane (one load beside the q
    // loads, not one dependent load per pair): lane i holds page id_base + i
    int id_base = p_begin;
    auto load_ids = [&](int base) {
      const int lp = base + lane;
      return lp < p_end ? bt[lp] : -1;
    };
    int ids = load_ids(id_base);
    // the pair at lp0: its blocks (bad ids read page 0 and are masked), its
    // page limit for the masked path, and whether it needs no mask at all
    // (lp0 - id_base is even and below 64: both pages are in `ids`)
    struct PairAt {
      const uint8_t* blk0;
      const uint8_t* blk1;
      int pe;
      bool interior;
    };
    auto pair_at = [&](int lp0) {
      const bool has1 = lp0 + 1 < p_end;
      int pg0 = __builtin_amdgcn_readlane(ids, lp0 - id_base);
      int pg1 = has1 ? __builtin_amdgcn_readlane(ids, lp0 + 1 - id_base) : pg0;
      const bool ok0 = pg0 >= 0 && pg0 < npg;
      const bool ok1 = pg1 >= 0 && pg1 < npg;
      if (!ok0) pg0 = 0;
      if (!ok1) pg1 = pg0;
      const int L0 = lp0 * kPage, L1 = (lp0 + 2) * kPage;
      // a chunk's queries mask the newer positions: every prefill pair is masked
      const bool interior =
          p.chunk == 1 && has1 && ok0 && ok1 && ((L1 <= n_sink) || (L0 >= ring0 && L1 <= ring0 + n_rec));
      return PairAt{block_ptr(p.bf16_pages, pg0, p.n_kv, kv, kBf16BlockBytes),
                    block_ptr(p.bf16_pages, pg1, p.n_kv, kv, kBf16BlockBytes), ok0 ? (ok1 ? p_end : lp0 + 1) : lp0,
                    interior};
    };
    PairAt pa = pair_at(p_begin);
    Bf16PairData cur = bf16_pair_load(pa.blk0, pa.blk1);
    for (int lp0 = p_begin; lp0 < p_end; lp0 += 2) {
      const bool more = lp0 + 2 < p_end;
      PairAt pn = pa;
      Bf16PairData nxt;
      if (more) {
        if (lp0 + 2 >= id_base + 64) {  // the next 64 page ids
          id_base += 64;
          ids = load_ids(id_base);
        }
        pn = pair_at(lp0 + 2);
        if constexpr (PREFETCH) nxt = bf16_pair_load(pn.blk0, pn.blk1);
      }
      if (pa.interior)
        bf16_pair<false>(p, cur, lp0, p_end, n_sink, ring0, n_rec, T, qpos, bq, m_run, l_run, acc);
      else
        bf16_pair<true>(p, cur, lp0, pa.pe, n_sink, ring0, n_rec, T, qpos, bq, m_run, l_run, acc);
      if (more) {
        if constexpr (PREFETCH)
          cur = nxt;
        else
          cur = bf16_pair_load(pn.blk0, pn.blk1);
      }
      pa = pn;
    }
  }
  const int S = p.splits_int2 + p.splits_bf16;
  const float l = sum_across_quads(l_run);
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int h = 4 * qd + r;
    if (h < p.g_real) {
      float* dst = p.partial + (((int64_t)b * p.n_q + kv * p.g + h0 + h) * S + split) * kPartialStride;
#pragma unroll
      for (int kt = 0; kt < 8; ++kt) dst[2 + 8 * ln + kt] = acc[kt][r];
    }
  }
  if (qd == 0 && ln < p.g_real) {
    float* dst = p.partial + (((int64_t)b * p.n_q + kv * p.g + h0 + ln) * S + split) * kPartialStride;
    dst[0] = m_run;
    dst[1] = l;
  }
}

// CT 16-row tiles per wavefront, W wavefronts per work item (tile_split).  One
// tile fits 4 wavefronts per SIMD (at most 126 VGPRs); two tiles, which share
// the unpacked codes, 3 on one-wavefront items (at 32-channel groups with a
// few spilled registers: measured 8 % faster than 2 without them); four 2.  Wavefronts of one item share the staged pages.  LDS per
// item: each wavefront's p and the staging ring (three slots for one
// wavefront, four when shared).
// BX (small grids, W = 1): the grid's last batch n_kv splits_bf16 work groups
// run the bf16 region, one split each (its pairs not prefetched), beside the
// INT2 items.  The kernel then holds the bf16 item's registers (208 VGPRs):
// two wavefronts per SIMD, all that a grid this form is chosen for needs.
template <int NG, int MB, int CT, int W, bool BX = false>
__global__ __launch_bounds__(64 * W) __attribute__((amdgpu_waves_per_eu(BX ? 2 : (CT == 1 ? 4 : (CT == 2 && W == 1 ? 3 : (CT == 2 || CT == 4 ? 2 : 1))), 8))) void
decode_int2(DecodeParams p) {
  __shared__ __attribute__((aligned(16))) float p_lds[W][(16 * CT / NG) * 32];
  __shared__ __attribute__((aligned(16))) uint8_t stage[(W == 1 ? 6 : 8) * Int2Layout{NG, MB}.bytes()];
  constexpr bool kWide = CT * (4 / NG) == 4;
  __shared__ __attribute__((aligned(16))) uint8_t edge_lds[kWide ? W * 2 * Int2Layout{NG, MB}.bytes() : 16];
  // XCD-aware order: blocks go to the eight XCDs in turn (block i to XCD
  // i % 8).  With a multiple of 8 (request, KV head) pairs every split of pair
  // bk runs on XCD bk % 8, the XCD of the prologue's and the combine's block
  // bk, so its q operands and partial rows pass through one L2; in time the
  // items still come pair by pair, as in the plain order.
  const int item = blockIdx.x;
  const int S = p.splits_int2, bkn = p.batch * p.n_kv;
  if constexpr (BX) {
    static_assert(W == 1, "bf16 items are one wavefront");
    if (item >= bkn * S) {
      const int e = item - bkn * S, pair = e / p.splits_bf16;
      bf16_item<false>(p, pair / p.n_kv, pair % p.n_kv, S + e % p.splits_bf16, 0);
      return;
    }
  }
  int split, bk;
  if ((bkn & 7) == 0) {
    const int j = item >> 3;
    split = j % S;
    bk = 8 * (j / S) + (item & 7);
  } else {
    split = item % S;
    bk = item / S;
  }
  float* pl = p_lds[W > 1 ? threadIdx.x >> 6 : 0];
  uint8_t* el = edge_lds + (kWide && W > 1 ? (threadIdx.x >> 6) : 0) * (kWide ? 2 * Int2Layout{NG, MB}.bytes() : 0);
  if constexpr (NG == 4 && CT == 4) {
    // a wide wavefront whose last tile holds no head (12 heads in 16 rows)
    // skips that tile's logits
    const int last = (W > 1 ? __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6)) * CT : 0) + CT - 1;
    if (4 * last >= p.g) {
      int2_item<NG, MB, CT, W, 0>(p, bk / p.n_kv, bk % p.n_kv, split, pl, stage, el);
      return;
    }
  }
  if constexpr (NG == 2) {
    // a 64-channel-group tile spans two head quads; when the second quad of
    // this wavefront's last tile holds no head (g % 8 <= 4), the loop skips
    // its logits (decided once per wavefront: the tile index is uniform)
    const int last = (W > 1 ? __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6)) * CT : 0) + CT - 1;
    if (8 * last + 4 >= p.g) {
      int2_item<NG, MB, CT, W, 1>(p, bk / p.n_kv, bk % p.n_kv, split, pl, stage, el);
      return;
    }
  }
  int2_item<NG, MB, CT, W, 4 / NG>(p, bk / p.n_kv, bk % p.n_kv, split, pl, stage, el);
}

// items: (request, KV head, query of the launch, bf16 split)
__global__ __launch_bounds__(64) void decode_bf16(DecodeParams p) {
  const int item = blockIdx.x;
  const int n_c = p.g / p.g_real;
  const int sb = item % p.splits_bf16;
  const int c = (item / p.splits_bf16) % n_c;
  const int bk = item / p.splits_bf16 / n_c;
  bf16_item<false>(p, bk / p.n_kv, bk % p.n_kv, p.splits_int2 + sb, c);
}

// ---------------------------------------------------------------------------
// combine: bf16 region (when its splits fit the block), LSE merge, R_V^T on
// the INT2 part, normalisation
// ---------------------------------------------------------------------------
// One block of eight wavefronts per (request, KV head), in two sides that run
// side by side.  Wavefronts 0-3 run the bf16 region (with bf16_in_combine:
// bf16 split w, at most four, its partial left beside the INT2 splits' ones)
// while wavefronts 4-7 stage R_V and merge the INT2 splits of query heads
// 0-3.  After a barrier, wavefront 4 + w applies R_V^T to the INT2 part of
// head w (then w + 4, ...) and wavefront w merges that head's bf16 splits;
// the INT2 side hands its part over through LDS and wavefront w combines the
// two.  Lane i owns output channels i and i + 64, so no step needs a
// block-wide reduction; the first 32 partial rows of a merge are loaded at
// once, behind the split maxima.  R_V is staged in LDS with a row stride of
// 129 floats: lane i reading rows i and i + 64 at column k hits bank
// (i + k) % 32, no conflicts.
constexpr int kRvStride = kHeadDim + 1;
constexpr int kCombineRows = 32;

// maximum / sum over the wavefront, in every lane: rows by DPP rotations, then
// the row pairs by permlane swaps (no LDS round trips)
__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int n = 1; n < 16; n <<= 1) x = fmaxf(x, __builtin_bit_cast(float, lane_ror(__builtin_bit_cast(uint32_t, x), n)));
  uint32_t a = __builtin_bit_cast(uint32_t, x), b = a;
  swap_rows<false>(a, b);
  x = fmaxf(__builtin_bit_cast(float, a), __builtin_bit_cast(float, b));
  a = b = __builtin_bit_cast(uint32_t, x);
  swap_rows<true>(a, b);
  return fmaxf(__builtin_bit_cast(float, a), __builtin_bit_cast(float, b));
}
__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int n = 1; n < 16; n <<= 1) x += __builtin_bit_cast(float, lane_ror(__builtin_bit_cast(uint32_t, x), n));
  uint32_t a = __builtin_bit_cast(uint32_t, x), b = a;
  swap_rows<false>(a, b);
  x = __builtin_bit_cast(float, a) + __builtin_bit_cast(float, b);
  a = b = __builtin_bit_cast(uint32_t, x);
  swap_rows<true>(a, b);
  return __builtin_bit_cast(float, a) + __builtin_bit_cast(float, b);
}
__device__ __forceinline__ float lane_value(float x, int l) {
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), l));
}

// rows [u0, u1) of one chunk of 64 splits, weights held by lanes u of `wt`:
// acc0 / acc1 += w_u row_u[lane] / row_u[lane + 64]
__device__ __forceinline__ void weighted_rows(const float* rows, float wt, int u0, int u1, float& acc0,
                                              float& acc1) {
  const int lane = threadIdx.x & 63;
  int u = u0;
  for (; u + 8 <= u1; u += 8) {
    float x0[8], x1[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      x0[k] = rows[(u + k) * kPartialStride + 2 + lane];
      x1[k] = rows[(u + k) * kPartialStride + 2 + 64 + lane];
    }
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const float wk = lane_value(wt, u + k);
      acc0 = fmaf(wk, x0[k], acc0);
      acc1 = fmaf(wk, x1[k], acc1);
    }
  }
  for (; u < u1; ++u) {
    const float wk = lane_value(wt, u);
    acc0 = fmaf(wk, rows[u * kPartialStride + 2 + lane], acc0);
    acc1 = fmaf(wk, rows[u * kPartialStride + 2 + 64 + lane], acc1);
  }
}

// log-sum-exp merge of the partial rows [s0, s1) of one head (base: its first
// partial row), by one wavefront: M = their largest max, L = sum 2^(m_s - M)
// l_s, acc = sum 2^(m_s - M) o_s (lane i: channels i and i + 64); M = -inf,
// L = acc = 0 when no row saw a token
__device__ void merge_splits(const float* base, int s0, int s1, float& M, float& L, float& a0, float& a1) {
  const int lane = threadIdx.x & 63;
  const int n = s1 - s0;
  M = kNegInf;
  L = a0 = a1 = 0.f;
  if (n <= 0) return;
  base += (int64_t)s0 * kPartialStride;
  // split maxima first, then the first rows, so that the max reduction waits
  // only for the former
  const float ms = lane < n ? base[lane * kPartialStride] : kNegInf;
  const float ls = lane < n ? base[lane * kPartialStride + 1] : 0.f;
  float m = ms;
  for (int s = lane + 64; s < n; s += 64) m = fmaxf(m, base[s * kPartialStride]);
  const int n0 = min(n, kCombineRows);
  float x0[kCombineRows], x1[kCombineRows];
#pragma unroll
  for (int k = 0; k < kCombineRows; ++k) {
    x0[k] = k < n0 ? base[k * kPartialStride + 2 + lane] : 0.f;
    x1[k] = k < n0 ? base[k * kPartialStride + 2 + 64 + lane] : 0.f;
  }
  M = wave_max(m);
  if (M == kNegInf) return;
  // a split without tokens has m = -inf and zero rows: weight 0
  const float wt0 = ms == kNegInf ? 0.f : exp2f(ms - M);
  float l = wt0 * ls;
#pragma unroll
  for (int k = 0; k < kCombineRows; ++k) {
    const float wk = lane_value(wt0, k);  // 0 past n
    a0 = fmaf(wk, x0[k], a0);
    a1 = fmaf(wk, x1[k], a1);
  }
  // the rest of the first 64 splits, then further chunks of 64
  for (int c0 = 0; c0 < n; c0 += 64) {
    float wt = wt0;
    if (c0 > 0) {
      const int s = c0 + lane;
      wt = 0.f;
      if (s < n) {
        const float mc = base[s * kPartialStride];
        wt = mc == kNegInf ? 0.f : exp2f(mc - M);
        l = fmaf(wt, base[s * kPartialStride + 1], l);
      }
    }
    weighted_rows(base + (int64_t)c0 * kPartialStride, wt, c0 == 0 ? n0 : 0, min(64, n - c0), a0, a1);
  }
  L = wave_sum(l);
}

__global__ __launch_bounds__(512) void decode_combine(DecodeParams p) {
  __shared__ float rv[kHeadDim * kRvStride];
  __shared__ __attribute__((aligned(16))) float aint[4][kHeadDim];  // INT2 part before R_V^T
  __shared__ float xch[4][kHeadDim + 2];                            // INT2 part, its M and L
  const int bk = blockIdx.x;
  const int b = bk / p.n_kv, kv = bk % p.n_kv;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, wl = w & 3;
  const bool int2_side = w >= 4;
  const int S = p.splits_int2 + p.splits_bf16, SI = p.splits_int2;
  // R_V null: the output stays in the rotated basis (R_V^T folded into the
  // output projection), and so does the bf16 region's V
  const bool rot = SI > 0 && p.r_v;
  auto base_of = [&](int h) { return p.partial + ((int64_t)b * p.n_q + kv * p.g + h) * S * kPartialStride; };
  float Mi = kNegInf, Li = 0.f, ai0 = 0.f, ai1 = 0.f;  // INT2 side: head h0 + wl
  if (int2_side) {
    if (rot) stage_matrix256<kRvStride>(p.r_v + (int64_t)kv * kHeadDim * kHeadDim, rv, threadIdx.x - 256);
    if (wl < p.g) merge_splits(base_of(wl), 0, SI, Mi, Li, ai0, ai1);
  } else if (p.bf16_in_combine && wl < p.splits_bf16) {
    bf16_item<true>(p, b, kv, SI + wl, 0);
  }
  __syncthreads();  // R_V staged; the bf16 partials written by this block are visible to it
  for (int h0 = 0; h0 < p.g; h0 += 4) {  // same trip count in every wavefront
    const int h = h0 + wl;
    float Mb = kNegInf, Lb = 0.f, ab0 = 0.f, ab1 = 0.f;
    if (h < p.g) {
      if (int2_side) {
        if (h0 > 0) merge_splits(base_of(h), 0, SI, Mi, Li, ai0, ai1);
        // R_V^T on the INT2 part: out_j = sum_k aint_k R_V[j][k]
        float r0 = ai0, r1 = ai1;
        if (rot) {
          aint[wl][lane] = ai0;
          aint[wl][lane + 64] = ai1;
          // the wavefront's own LDS writes, read back by its other lanes (LDS
          // operations of one wavefront complete in order)
          __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
          __builtin_amdgcn_wave_barrier();
          __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
          // 32 k at a time: every LDS read of a batch is issued before its
          // FMAs (one LDS latency per batch, not one per read), two
          // accumulators per output
          float r0b = 0.f, r1b = 0.f;
          r0 = r1 = 0.f;
          const float* row0 = rv + lane * kRvStride;
          const float* row1 = rv + (lane + 64) * kRvStride;
#pragma unroll
          for (int k0 = 0; k0 < kHeadDim; k0 += 32) {
            float4 a[8];
            float x0[32], x1[32];
#pragma unroll
            for (int i = 0; i < 8; ++i) a[i] = *(const float4*)&aint[wl][k0 + 4 * i];
#pragma unroll
            for (int i = 0; i < 32; ++i) {
              x0[i] = row0[k0 + i];
              x1[i] = row1[k0 + i];
            }
#pragma unroll
            for (int i = 0; i < 8; ++i) {
              r0 = fmaf(a[i].x, x0[4 * i], r0);
              r1 = fmaf(a[i].x, x1[4 * i], r1);
              r0b = fmaf(a[i].y, x0[4 * i + 1], r0b);
              r1b = fmaf(a[i].y, x1[4 * i + 1], r1b);
              r0 = fmaf(a[i].z, x0[4 * i + 2], r0);
              r1 = fmaf(a[i].z, x1[4 * i + 2], r1);
              r0b = fmaf(a[i].w, x0[4 * i + 3], r0b);
              r1b = fmaf(a[i].w, x1[4 * i + 3], r1b);
            }
          }
          r0 += r0b;
          r1 += r1b;
        }
        xch[wl][lane] = r0;
        xch[wl][lane + 64] = r1;
        if (lane == 0) {
          xch[wl][kHeadDim] = Mi;
          xch[wl][kHeadDim + 1] = Li;
        }
      } else {
        merge_splits(base_of(h), SI, S, Mb, Lb, ab0, ab1);
      }
    }
    __syncthreads();  // the INT2 part of heads h0 .. h0 + 3 is in xch
    if (!int2_side && h < p.g) {
      const float mi = xch[wl][kHeadDim], li = xch[wl][kHeadDim + 1];
      const float M = fmaxf(mi, Mb);
      float* o = p.out + q_row(p, b, kv, h);
      if (M == kNegInf) {  // no token at all
        o[lane] = 0.f;
        o[lane + 64] = 0.f;
      } else {
        const float wi = mi == kNegInf ? 0.f : exp2f(mi - M), wb = Mb == kNegInf ? 0.f : exp2f(Mb - M);
        const float L = wi * li + wb * Lb;
        o[lane] = (wi * xch[wl][lane] + wb * ab0) / L;
        o[lane + 64] = (wi * xch[wl][lane + 64] + wb * ab1) / L;
      }
    }
    __syncthreads();  // xch is free again
  }
}

// ---------------------------------------------------------------------------
// combine on small grids: one work group per (request, KV head, query head)
// ---------------------------------------------------------------------------
// With one request (say) the form above runs eight work groups, each a chain
// of dependent loads.  Here the bf16 splits have run inside the INT2 kernel's
// grid, and each query head takes a work group of nine wavefronts: wavefront w
// < 8 merges the INT2 splits [w SI / 8, (w + 1) SI / 8) of the head (16 rows at
// 128 splits: one batch of loads), R_V's loads in flight meanwhile and its LDS
// stores after; wavefront 8 merges the bf16 splits.  The eight INT2 parts are
// joined in LDS, and R_V^T is spread over the eight wavefronts: output channel
// 16 w + lane / 4, a quarter of k per lane, summed over the lane quad.
constexpr int kHeadMergeWaves = 8;

__global__ __launch_bounds__(64 * (kHeadMergeWaves + 1)) void decode_combine_head(DecodeParams p) {
  __shared__ float rv[kHeadDim * kRvStride];
  __shared__ float part[kHeadMergeWaves][kHeadDim + 2];  // each INT2 range: rows, M, L
  __shared__ float bpart[kHeadDim + 2];                  // the bf16 splits: rows, M, L
  __shared__ float ajoin[kHeadDim];                      // the joined INT2 part
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  // XCD-aware order, as in the INT2 kernel: the work groups of pair bk run on
  // XCD bk % 8, where that pair's partial rows were written
  const int bkn = p.batch * p.n_kv, g = p.g, item = blockIdx.x;
  int bk, h;
  if ((bkn & 7) == 0) {
    const int j = item >> 3;
    h = j % g;
    bk = 8 * (j / g) + (item & 7);
  } else {
    h = item % g;
    bk = item / g;
  }
  const int b = bk / p.n_kv, kv = bk % p.n_kv;
  const int S = p.splits_int2 + p.splits_bf16, SI = p.splits_int2;
  const bool rot = SI > 0 && p.r_v;
  const float* base = p.partial + ((int64_t)b * p.n_q + kv * g + h) * S * kPartialStride;
  float M, L, a0, a1;
  if (w < kHeadMergeWaves) {
    constexpr int kT = 64 * kHeadMergeWaves, kPer = kHeadDim * kHeadDim / 4 / kT;
    float4 rvv[kPer];
    const float4* R = (const float4*)(p.r_v + (int64_t)kv * kHeadDim * kHeadDim);
    if (rot) {
#pragma unroll
      for (int k = 0; k < kPer; ++k) rvv[k] = R[threadIdx.x + kT * k];
    }
    merge_splits(base, (int)((int64_t)w * SI / kHeadMergeWaves), (int)((int64_t)(w + 1) * SI / kHeadMergeWaves), M,
                 L, a0, a1);
    part[w][lane] = a0;
    part[w][lane + 64] = a1;
    if (lane == 0) {
      part[w][kHeadDim] = M;
      part[w][kHeadDim + 1] = L;
    }
    if (rot) {
#pragma unroll
      for (int k = 0; k < kPer; ++k) {
        const int e = threadIdx.x + kT * k;
        float* d = rv + (e >> 5) * kRvStride + 4 * (e & 31);
        d[0] = rvv[k].x;
        d[1] = rvv[k].y;
        d[2] = rvv[k].z;
        d[3] = rvv[k].w;
      }
    }
  } else {
    merge_splits(base, SI, S, M, L, a0, a1);
    bpart[lane] = a0;
    bpart[lane + 64] = a1;
    if (lane == 0) {
      bpart[kHeadDim] = M;
      bpart[kHeadDim + 1] = L;
    }
  }
  __syncthreads();  // the nine parts and R_V are in LDS
  // join the INT2 ranges: mi their largest max, each weighted by 2^(M_w - mi)
  // (0 for a range without tokens)
  float mi = kNegInf;
#pragma unroll
  for (int r = 0; r < kHeadMergeWaves; ++r) mi = fmaxf(mi, part[r][kHeadDim]);
  float wts[kHeadMergeWaves], li = 0.f;
#pragma unroll
  for (int r = 0; r < kHeadMergeWaves; ++r) {
    const float mr = part[r][kHeadDim];
    wts[r] = mr == kNegInf ? 0.f : exp2f(mr - mi);
    li = fmaf(wts[r], part[r][kHeadDim + 1], li);
  }
  if (w < kHeadMergeWaves && lane < kHeadDim / kHeadMergeWaves) {
    const int k = (kHeadDim / kHeadMergeWaves) * w + lane;
    float a = 0.f;
#pragma unroll
    for (int r = 0; r < kHeadMergeWaves; ++r) a = fmaf(wts[r], part[r][k], a);
    ajoin[k] = a;
  }
  __syncthreads();  // the joined INT2 part is in LDS
  if (w >= kHeadMergeWaves) return;
  const int j = (kHeadDim / kHeadMergeWaves) * w + (lane >> 2), kq = lane & 3;
  float r;
  if (rot) {
    // out_j = sum_k a_k R_V[j][k]: lane quarter kq of k, read from k offset
    // 8 kq on (the 32 lanes of a half-wavefront then hit 32 distinct banks)
    const float* row = rv + j * kRvStride + 32 * kq;
    const float* av = ajoin + 32 * kq;
    float x[32], y[32];
#pragma unroll
    for (int i = 0; i < 32; ++i) {
      const int kk = (i + 8 * kq) & 31;
      x[i] = row[kk];
      y[i] = av[kk];
    }
    float r0 = 0.f, r1 = 0.f;
#pragma unroll
    for (int i = 0; i < 32; i += 2) {
      r0 = fmaf(y[i], x[i], r0);
      r1 = fmaf(y[i + 1], x[i + 1], r1);
    }
    r = r0 + r1;
    // sum over the lane quad (DPP quad permutations [1,0,3,2] and [2,3,0,1])
    r += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, r), 0xb1, 0xf, 0xf, false));
    r += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, r), 0x4e, 0xf, 0xf, false));
  } else {
    r = ajoin[j];
  }
  if (kq == 0) {
    const float mb = bpart[kHeadDim], lb = bpart[kHeadDim + 1];
    const float Mx = fmaxf(mi, mb);
    float* o = p.out + q_row(p, b, kv, h);
    if (Mx == kNegInf) {  // no token at all
      o[j] = 0.f;
    } else {
      const float wi = mi == kNegInf ? 0.f : exp2f(mi - Mx), wb = mb == kNegInf ? 0.f : exp2f(mb - Mx);
      o[j] = (wi * r + wb * bpart[j]) / (wi * li + wb * lb);
    }
  }
}

template <int NG, int MB, int CT, int W>
hipError_t launch_decode_t(const DecodeParams& p, hipStream_t stream, hipEvent_t ev_start, hipEvent_t ev_stop,
                           const ArgTables& tabs) {
  const int bkn = p.batch * p.n_kv;
  // the event pair brackets the dominant kernel: the INT2 stream when there is
  // one, else the bf16 stream.  (Running the bf16 kernel on a second stream
  // beside the INT2 kernel was measured slower: its wavefronts take slots from
  // the INT2 kernel's full rounds.  Up to four bf16 splits run inside the
  // combine instead.)
  const bool int2 = p.splits_int2 > 0;
  // the small-grid form: one-wavefront INT2 items only
  if (p.small_grid && (W != 1 || !int2 || p.splits_bf16 < 1)) return hipErrorInvalidValue;
  auto mark = [&](hipEvent_t ev) { return ev ? hipEventRecord(ev, stream) : hipSuccess; };
  hipError_t e = hipSuccess;
  if (int2) {
    if (p.has_step)
      hipLaunchKernelGGL((decode_prologue<NG, MB, CT * W, true>), dim3((1 + p.split_writes) * bkn), dim3(256), 0,
                         stream, p, tabs);
    else
      hipLaunchKernelGGL((decode_prologue<NG, MB, CT * W, false>), dim3(bkn), dim3(256), 0, stream, p, tabs);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    if ((e = mark(ev_start)) != hipSuccess) return e;
    if constexpr (W == 1) {
      if (p.small_grid) {
        hipLaunchKernelGGL((decode_int2<NG, MB, CT, 1, true>), dim3(bkn * (p.splits_int2 + p.splits_bf16)), dim3(64),
                           0, stream, p);
        if ((e = hipGetLastError()) != hipSuccess) return e;
        if ((e = mark(ev_stop)) != hipSuccess) return e;
        hipLaunchKernelGGL(decode_combine_head, dim3(bkn * p.g), dim3(64 * (kHeadMergeWaves + 1)), 0, stream, p);
        return hipGetLastError();
      }
    }
    hipLaunchKernelGGL((decode_int2<NG, MB, CT, W>), dim3(bkn * p.splits_int2), dim3(64 * W), 0, stream, p);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    if ((e = mark(ev_stop)) != hipSuccess) return e;
  }
  if (p.splits_bf16 > 0 && !p.bf16_in_combine) {
    if (!int2 && (e = mark(ev_start)) != hipSuccess) return e;
    hipLaunchKernelGGL(decode_bf16, dim3(bkn * (p.g / p.g_real) * p.splits_bf16), dim3(64), 0, stream, p);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    if (!int2 && (e = mark(ev_stop)) != hipSuccess) return e;
  }
  hipLaunchKernelGGL(decode_combine, dim3(bkn), dim3(512), 0, stream, p);
  return hipGetLastError();
}

// One query block of a chunked prefill: W = p.ct tiles, one wavefront each.
template <int NG, int MB, int W>
hipError_t launch_prefill_t(const DecodeParams& p, hipStream_t stream, hipEvent_t ev_start, hipEvent_t ev_stop) {
  const int bkn = p.batch * p.n_kv;
  auto mark = [&](hipEvent_t ev) { return ev ? hipEventRecord(ev, stream) : hipSuccess; };
  hipError_t e = hipSuccess;
  hipLaunchKernelGGL((prefill_prologue<NG>), dim3(bkn), dim3(256), 0, stream, p);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if ((e = mark(ev_start)) != hipSuccess) return e;
  // 32-channel groups: wide items, four tiles (16 kernel heads) per
  // wavefront.  At 64-channel groups one tile per wavefront, four per SIMD,
  // measured 5 % faster than two-tile wide wavefronts at two per SIMD.
  constexpr int kCt = NG == 4 ? 4 : 1;
  hipLaunchKernelGGL((decode_int2<NG, MB, kCt, W / kCt>), dim3(bkn * p.splits_int2), dim3(64 * (W / kCt)), 0, stream,
                     p);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if ((e = mark(ev_stop)) != hipSuccess) return e;
  hipLaunchKernelGGL(decode_bf16, dim3(bkn * (p.g / p.g_real) * p.splits_bf16), dim3(64), 0, stream, p);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL(decode_combine, dim3(bkn), dim3(512), 0, stream, p);
  return hipGetLastError();
}

template <int MB>
hipError_t launch_prefill_mb(const DecodeParams& p, hipStream_t stream, hipEvent_t ev_start, hipEvent_t ev_stop) {
  if (p.ng == 4) {
    if (p.ct == 4) return launch_prefill_t<4, MB, 4>(p, stream, ev_start, ev_stop);
    if (p.ct == 8) return launch_prefill_t<4, MB, 8>(p, stream, ev_start, ev_stop);
    if (p.ct == 16) return launch_prefill_t<4, MB, 16>(p, stream, ev_start, ev_stop);
  } else if (p.ng == 2) {
    if (p.ct == 4) return launch_prefill_t<2, MB, 4>(p, stream, ev_start, ev_stop);
    if (p.ct == 8) return launch_prefill_t<2, MB, 8>(p, stream, ev_start, ev_stop);
    if (p.ct == 16) return launch_prefill_t<2, MB, 16>(p, stream, ev_start, ev_stop);
  }
  return hipErrorInvalidValue;
}

template <int MB>
hipError_t launch_decode_mb(const DecodeParams& p, hipStream_t stream, hipEvent_t ev_start, hipEvent_t ev_stop,
                            const ArgTables& tabs) {
  // p.ct = 16-row tiles of a (request, KV head), spread as tile_split says
  const TileSplit ts = tile_split(p.ct);
  const int key = ts.ct * 10 + ts.w;
  if (ts.ct * ts.w != p.ct) return hipErrorInvalidValue;
  if (p.ng == 4) {
    if (key == 11) return launch_decode_t<4, MB, 1, 1>(p, stream, ev_start, ev_stop, tabs);
    if (key == 21) return launch_decode_t<4, MB, 2, 1>(p, stream, ev_start, ev_stop, tabs);
    if (key == 13) return launch_decode_t<4, MB, 1, 3>(p, stream, ev_start, ev_stop, tabs);
    if (key == 22) return launch_decode_t<4, MB, 2, 2>(p, stream, ev_start, ev_stop, tabs);
    if (key == 41) return launch_decode_t<4, MB, 4, 1>(p, stream, ev_start, ev_stop, tabs);
  } else if (p.ng == 2) {
    if (key == 11) return launch_decode_t<2, MB, 1, 1>(p, stream, ev_start, ev_stop, tabs);
    if (key == 21) return launch_decode_t<2, MB, 2, 1>(p, stream, ev_start, ev_stop, tabs);
  }
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_decode(const DecodeParams& p, hipStream_t stream, hipEvent_t ev_start, hipEvent_t ev_stop,
                         const ArgTables* tabs) {
  static const ArgTables kNoTables{};
  const ArgTables& t = tabs ? *tabs : kNoTables;
  if (p.mb == 4) return launch_decode_mb<4>(p, stream, ev_start, ev_stop, t);
  if (p.mb == 2) return launch_decode_mb<2>(p, stream, ev_start, ev_stop, t);
  return hipErrorInvalidValue;
}

hipError_t launch_prefill(const DecodeParams& p, hipStream_t stream, hipEvent_t ev_start, hipEvent_t ev_stop) {
  if (p.mb == 4) return launch_prefill_mb<4>(p, stream, ev_start, ev_stop);
  if (p.mb == 2) return launch_prefill_mb<2>(p, stream, ev_start, ev_stop);
  return hipErrorInvalidValue;
}

static size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

size_t decode_workspace_bytes(int batch, int n_q, int n_kv, int ct, int splits_total) {
  const size_t bkn = (size_t)batch * n_kv;
  return align256(bkn * ct * 3 * 2 * 64 * 4 * sizeof(uint32_t)) + align256(bkn * (1 + 16 * ct) * sizeof(float)) +
         align256((size_t)batch * n_q * splits_total * kPartialStride * sizeof(float)) +
         align256((size_t)batch * sizeof(int32_t));
}

void decode_workspace_carve(DecodeParams& p, void* ws) {
  const size_t bkn = (size_t)p.batch * p.n_kv;
  uint8_t* w = (uint8_t*)ws;
  p.qb = (uint32_t*)w;
  w += align256(bkn * p.ct * 3 * 2 * 64 * 4 * sizeof(uint32_t));
  p.qaux = (float*)w;
  w += align256(bkn * (1 + 16 * p.ct) * sizeof(float));
  p.partial = (float*)w;
  w += align256((size_t)p.batch * p.n_q * (p.splits_int2 + p.splits_bf16) * kPartialStride * sizeof(float));
  p.ctx_w = (int32_t*)w;
}


// ---- The allocation-free decode's workspace ----
// For callers that cannot allocate device memory (code under graph capture,
// serving loops, harnesses that forbid it): the split-K workspace of
// oscar_decode_attn_noalloc lives in this array.  Each GPU the library runs on
// holds its own copy for the life of the process.  In host code the array's
// name is not a device address: the address is looked up per device with
// hipGetSymbolAddress and only that address is handed to kernels.  Every byte
// a launch reads is written earlier in the same launch, so nothing is cleared;
// calls that overlap on one GPU share the array and race.
static __device__ __align__(256) uint8_t scratch[kDecodeScratchBytes];

namespace {
constexpr int kScratchMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_addr[kScratchMaxDevices] = {};
}  // namespace

hipError_t decode_scratch(hipStream_t stream, void** ptr, size_t* bytes) {
  int dev = -1;
  hipError_t e = stream ? hipStreamGetDevice(stream, &dev) : hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kScratchMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_addr[dev]) {
    // look the address up with the stream's device current
    int cur = -1;
    if ((e = hipGetDevice(&cur)) != hipSuccess) return e;
    if (cur != dev && (e = hipSetDevice(dev)) != hipSuccess) return e;
    void* addr = nullptr;
    e = hipGetSymbolAddress(&addr, HIP_SYMBOL(scratch));
    if (cur != dev) {
      const hipError_t back = hipSetDevice(cur);
      if (e == hipSuccess) e = back;
    }
    if (e != hipSuccess) return e;
    if (!addr) return hipErrorInvalidSymbol;
    g_scratch_addr[dev] = addr;
  }
  *ptr = g_scratch_addr[dev];
  *bytes = kDecodeScratchBytes;
  return hipSuccess;
}

}  // namespace oscar
