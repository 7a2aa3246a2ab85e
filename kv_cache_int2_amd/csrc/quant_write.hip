// OSCAR write path for gfx950: rotate, clip, per-token asymmetric INT2 per
// channel group, pack into the paged INT2 blocks.
//
// [ES] "El sistema de servicio", write path: each token is rotated by the fixed
// calibrated rotation, clipped at the calibrated percentile threshold, and
// quantised to asymmetric INT2 per token with a group of channels sharing a
// scale and zero point.  [IT] 2.2.B: the history lives in INT2 after the fixed
// rotation and clip.
//
// The quantiser's decisions are taken on the exact rotated value x~ = x R (x
// bf16, R fp32), the precision a double-precision reference has:
//   s = fp16((mx - mn) / 3), z = fp16(mn) (or FP8 E4M3 in the lower-metadata
//   format), each one rounding to nearest-even; code = clamp(rint((x - z) / s),
//   0, 3) against the rounded s and z.
//
// Rotation as exact integer arithmetic on int8 MFMA.  Per token, x is taken as
// the integer X = rint(x 2^(28-E)) (2^E <= max|x| < 2^(E+1), |X| < 2^29); an
// entry below 2^(E-21) may be rounded, by at most half a unit.  R is the integer
// Y = rint(R 2^30) plus a residual digit lo = rint((R - Y 2^-30) 2^38).  X and
// Y are split into four balanced base-256 digits each (no bias); every digit
// pair of weight 256^1 and above, and the pair (top X digit, lo), is one
// v_mfma_i32_16x16x64_i8 chain with exact int32 sums (16 pairs), and the six
// weight classes are joined in fp64 (one rounding).  What separates that
// value from x R is bounded per token: the rounded entries, n 2^(E-29)
// max|R_ij|; the residual of R beyond lo, 2^(E+1) max_j sum_i |R_ij - Y_ij
// 2^-30 - lo_ij 2^-38|; the lower three X digits against R - Y 2^-30,
// 8421504 2^(E-28) max_j sum_i |R_ij - Y_ij 2^-30|; the omitted pair of
// weight 256^0, 128 2^(E-58) sum_i |D0_i| over the token's lowest X digit
// (zero when every entry is at least 2^(E-13)); and the fp64 join, 2^(E-52)
// max_j sum_i |R_ij|.  The bound also covers a double-precision reference's
// own sum, 128 2^-53 sum_i |x_i R_ij| <= 2^(E-45) max_j sum_i |R_ij|.
//
// Certification.  Each decision is checked in fp64 against that bound: z and
// s are taken only if the fp16 (or FP8) rounding is the same at both ends of
// the interval that holds the exact value (rounding is monotone), each code
// only if its t lies farther than the bound from a rounding boundary.  Tokens
// with non-finite values or max|x| below 2^-87, rotations with entries outside
// [-1.5, 1.5] or non-finite, and every decision the bound leaves open send
// their 16-token tile to the exact path: x R in fp64 on
// v_mfma_f64_16x16x4_f64 (bf16 and fp32 products are exact, sums fp64) and the
// quantiser in fp64 with IEEE division, the same arithmetic as a
// double-precision reference.
//
// Work decomposition: a work group of four wavefronts holds the digits of one
// (KV head, K or V) rotation in registers (wavefront w: output channels
// 32w..32w+31) and walks tiles of 16 tokens; each tile's slots and inputs are
// fetched while the tile before it is processed.  Per tile the 256 threads
// write the digits of the bf16 inputs to LDS, each wavefront runs 32 int8
// MFMAs per 16-channel tile and the epilogue for its channels, then wavefront
// 0 packs and stores the tile.
//
// Storage (per (page, KV head) block): K codes token-major (a token's 32 bytes
// are its own) with token-major scale/zero, V codes by token quad [4][128]
// bytes (byte j of quad q: channel j of tokens 4q..4q+3) with group-major
// scale/zero.  A V dword (4 channels of one quad) is written whole when the
// tile holds all 4 tokens of the quad, else merged with 32-bit atomic and/or,
// so tokens of one page may be written by different work groups or launches.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "oscar_internal.h"
#include "quant_common.h"

namespace oscar {
namespace {

typedef double f64x4 __attribute__((ext_vector_type(4)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kTok = 16;        // tokens per tile
constexpr int kWaves = 4;       // wavefronts per work group
constexpr int kThreads = 64 * kWaves;
constexpr int kClasses = 6;     // digit-pair weights 256^1 .. 256^6 (the 256^0 pair is omitted)
constexpr double kOmit = 128.0 * 0x1p-58;  // the omitted pair per unit of |D0|, times 2^-E
constexpr int kCodeRow = kHeadDim + 4;  // padded LDS row of a token's codes (no bank conflicts)
__device__ __forceinline__ float bf16_to_f32(uint32_t b) { return __builtin_bit_cast(float, b << 16); }

__device__ __forceinline__ i32x4 mfma_i8(u32x4 a, u32x4 b, i32x4 c) {
  return __builtin_amdgcn_mfma_i32_16x16x64_i8(__builtin_bit_cast(i32x4, a), __builtin_bit_cast(i32x4, b), c, 0, 0,
                                               0);
}

// byte k of each of u0..u3, in that order (v_perm_b32 picks bytes of {S0:S1})
__device__ __forceinline__ uint32_t gather_byte(uint32_t u0, uint32_t u1, uint32_t u2, uint32_t u3, int k) {
  const uint32_t sel = (uint32_t)k | ((uint32_t)(4 + k) << 8) | 0x0c0c0000u;
  const uint32_t p01 = __builtin_amdgcn_perm(u1, u0, sel);
  const uint32_t p23 = __builtin_amdgcn_perm(u3, u2, sel);
  return __builtin_amdgcn_perm(p23, p01, 0x05040100u);
}
// bytes 0 and 1 of each of u0..u3: (byte 0 of all four, byte 1 of all four)
__device__ __forceinline__ void gather_bytes01(uint32_t u0, uint32_t u1, uint32_t u2, uint32_t u3, uint32_t& b0,
                                               uint32_t& b1) {
  const uint32_t q01 = __builtin_amdgcn_perm(u1, u0, 0x05010400u);  // u0.b0 u1.b0 u0.b1 u1.b1
  const uint32_t q23 = __builtin_amdgcn_perm(u3, u2, 0x05010400u);
  b0 = __builtin_amdgcn_perm(q23, q01, 0x05040100u);
  b1 = __builtin_amdgcn_perm(q23, q01, 0x07060302u);
}

// Lane exchanges without LDS.  A wavefront is four rows of 16 lanes.
// dpp_ror: every lane takes the value of the lane n places around its row.
__device__ __forceinline__ uint32_t dpp_ror(uint32_t x, int n) {
  switch (n) {
    case 1: return (uint32_t)__builtin_amdgcn_mov_dpp((int)x, 0x121, 0xf, 0xf, false);
    case 2: return (uint32_t)__builtin_amdgcn_mov_dpp((int)x, 0x122, 0xf, 0xf, false);
    case 4: return (uint32_t)__builtin_amdgcn_mov_dpp((int)x, 0x124, 0xf, 0xf, false);
    default: return (uint32_t)__builtin_amdgcn_mov_dpp((int)x, 0x128, 0xf, 0xf, false);
  }
}
// maximum / sum over the 16 lanes of each row, in every lane (windows of 1, 2, 4, 8 lanes doubled)
__device__ __forceinline__ uint32_t row_max_u32(uint32_t x) {
#pragma unroll
  for (int n = 1; n < 16; n <<= 1) {
    const uint32_t y = dpp_ror(x, n);
    x = y > x ? y : x;
  }
  return x;
}
__device__ __forceinline__ int row_sum_i32(int x) {
#pragma unroll
  for (int n = 1; n < 16; n <<= 1) x += (int)dpp_ror((uint32_t)x, n);
  return x;
}
// v_permlane16_swap / v_permlane32_swap with x in both registers: the pair
// (first, second) holds, for each lane, the values of the two rows it is
// paired with: rows (0,1) and (2,3) for 16, rows (0,2) and (1,3) for 32.
// Written in asm: the compiler's builtins for them have handed back the first
// register for both results.  The s_nop 1 before gives the two wait states a
// swap needs after a VALU write of its operands; the one after gives the two a
// DPP read of a result needs (the compiler does not count an asm block as a
// VALU write).
struct RowPair {
  uint32_t a, b;
};
__device__ __forceinline__ RowPair swap16(uint32_t x) {
  RowPair r{x, x};
  asm volatile("s_nop 1\n\tv_permlane16_swap_b32 %0, %1\n\ts_nop 1" : "+v"(r.a), "+v"(r.b));
  return r;
}
__device__ __forceinline__ RowPair swap32(uint32_t x) {
  RowPair r{x, x};
  asm volatile("s_nop 1\n\tv_permlane32_swap_b32 %0, %1\n\ts_nop 1" : "+v"(r.a), "+v"(r.b));
  return r;
}
__device__ __forceinline__ double f64_of(uint32_t lo, uint32_t hi) {
  return __builtin_bit_cast(double, (uint64_t)lo | ((uint64_t)hi << 32));
}
// minimum and maximum over the four rows (same position in each row), in every lane
__device__ __forceinline__ void rows_minmax(double& mn, double& mx) {
  {
    const uint64_t un = __builtin_bit_cast(uint64_t, mn), ux = __builtin_bit_cast(uint64_t, mx);
    const RowPair nl = swap16((uint32_t)un), nh = swap16((uint32_t)(un >> 32));
    const RowPair xl = swap16((uint32_t)ux), xh = swap16((uint32_t)(ux >> 32));
    mn = __builtin_fmin(f64_of(nl.a, nh.a), f64_of(nl.b, nh.b));
    mx = __builtin_fmax(f64_of(xl.a, xh.a), f64_of(xl.b, xh.b));
  }
  {
    const uint64_t un = __builtin_bit_cast(uint64_t, mn), ux = __builtin_bit_cast(uint64_t, mx);
    const RowPair nl = swap32((uint32_t)un), nh = swap32((uint32_t)(un >> 32));
    const RowPair xl = swap32((uint32_t)ux), xh = swap32((uint32_t)(ux >> 32));
    mn = __builtin_fmin(f64_of(nl.a, nh.a), f64_of(nl.b, nh.b));
    mx = __builtin_fmax(f64_of(xl.a, xh.a), f64_of(xl.b, xh.b));
  }
}
// the value of row k of x, k = 0..3, in every lane (r[k])
__device__ __forceinline__ void rows_gather(uint32_t x, uint32_t r[4]) {
  const RowPair p = swap16(x);   // a: rows 0, 0, 2, 2   b: rows 1, 1, 3, 3
  const RowPair qa = swap32(p.a);  // a: row 0  b: row 2
  const RowPair qb = swap32(p.b);  // a: row 1  b: row 3
  r[0] = qa.a;
  r[1] = qb.a;
  r[2] = qa.b;
  r[3] = qb.b;
}

__device__ __forceinline__ uint16_t f32_to_f16_bits(float x) { return __builtin_bit_cast(uint16_t, (_Float16)x); }

// binary64 -> binary16 with one rounding to nearest even: round to odd into
// binary32 (24 bits, 13 more than binary16), then nearest even to binary16.
__device__ __forceinline__ uint32_t f16_bits_rn(double d) {
  const float f = (float)d;
  const double back = (double)f;
  uint32_t b = __builtin_bit_cast(uint32_t, f);
  if (back != d) {
    if (__builtin_fabs(back) > __builtin_fabs(d)) b -= 1u;  // the neighbour toward zero
    b |= 1u;
  }
  return f32_to_f16_bits(__builtin_bit_cast(float, b));
}

// The stored bits of a certified scale or zero, and the value the codes are
// taken against.
template <int MB>
__device__ __forceinline__ uint32_t meta_bits(double v) {
  if constexpr (MB == 4)
    return f16_bits_rn(v);
  else
    return f64_to_e4m3(v);
}
template <int MB>
__device__ __forceinline__ double meta_value(uint32_t bits) {
  if constexpr (MB == 4)
    return (double)__builtin_bit_cast(_Float16, (uint16_t)bits);
  else
    return e4m3_to_f64((uint8_t)bits);
}

struct alignas(16) TokInfo {
  double c8;       // unit of the lowest kept weight class: 2^(E-50)
  double bound;    // bound on |exact - fixed-point| (and a reference's own error) of every entry
  int exact;       // nonzero: the tile takes the exact path for this token
  int pad[3];
};

constexpr int kMaxTilesPerWg = 64;  // bounds the list of tiles sent to the exact path

struct Smem {
  // main loop, buffered so that one barrier per tile orders every access
  uint8_t xdig[2][4][2][4][kTok][16];  // by tile parity: x digits [digit][K half][lane quad][token][16 channels]
  TokInfo tok[3][kTok];                // by tile mod 3
  alignas(16) int32_t dst[3][kTok];    // by tile mod 3
  uint8_t codes[2][kTok][kCodeRow];    // by tile parity; the exact path uses [0]
  u32x4 rlo[kWaves][2][2][64];         // the residual digit of R: A operand of wavefront w, tile s, half h
  uint32_t flag[2][kWaves];            // by tile parity, per wavefront: some decision not certified
  double part[kTok][kWaves][2];        // per-wavefront group min/max (64-channel groups)
  uint32_t rbits[4];                   // float bits of the maxima over channels j of sum_i |R_ij - Y_ij 2^-30|,
                                       // sum_i |R_ij - Y_ij 2^-30 - lo_ij 2^-38|, sum_i |R_ij|, and of max |R_ij|
  uint32_t bad_r;                      // some entry of R is non-finite or outside [-1.5, 1.5]
  uint32_t fb_n;                       // tiles sent to the exact path, as offsets from the first tile
  uint16_t fb_list[kMaxTilesPerWg];
  // the exact path, after the main loop
  uint16_t xraw[kTok][kHeadDim];       // bf16 inputs of the tile
  alignas(16) int32_t dst_x[kTok];
  uint32_t szs[kTok][4];
  double xr[kTok][kHeadDim + 1];       // rotated values
};

// ---- the exact path for one tile: x R in fp64 on MFMA, quantiser in fp64 ----
typedef const float __attribute__((address_space(1))) * gfloat_ptr;

// f64 16x16x4 operands: A lane l -> A[l%16][l/16]; B lane l -> B[l/16][l%16];
// C lane l, element r -> C[4r + l/16][l%16].  Wavefront w: column tiles 2w, 2w+1.
// The B operands of the lane: R[4ks + l/16][16(2w+s) + l%16].  R is device
// global memory (read through that address space, so that LDS waits do not
// wait for these loads as well).
__device__ __forceinline__ void exact_load_r(const float* R, int lane, int wave, float rb[2][kHeadDim / 4]) {
  if (!R) return;
  const gfloat_ptr Rg = (gfloat_ptr)R;
  const int ln = lane & 15, qd = lane >> 4;
#pragma unroll
  for (int s = 0; s < 2; ++s)
#pragma unroll
    for (int ks = 0; ks < kHeadDim / 4; ++ks) rb[s][ks] = Rg[(4 * ks + qd) * kHeadDim + 16 * (2 * wave + s) + ln];
}

template <int NG, int MB>
__device__ __forceinline__ void exact_tile(Smem& S, const float* R, const float rb[2][kHeadDim / 4], double tau,
                                           int lane, int wave) {
  constexpr int G = kHeadDim / NG;
  const int ln = lane & 15, qd = lane >> 4;
  if (R) {
    // per column tile two interleaved accumulation chains (even and odd k steps), added at the end
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      f64x4 acc0 = f64x4{0.0, 0.0, 0.0, 0.0}, acc1 = f64x4{0.0, 0.0, 0.0, 0.0};
#pragma unroll
      for (int ks = 0; ks < kHeadDim / 4; ks += 2) {
        acc0 = __builtin_amdgcn_mfma_f64_16x16x4f64((double)bf16_to_f32(S.xraw[ln][4 * ks + qd]), (double)rb[s][ks],
                                                    acc0, 0, 0, 0);
        acc1 = __builtin_amdgcn_mfma_f64_16x16x4f64((double)bf16_to_f32(S.xraw[ln][4 * ks + 4 + qd]),
                                                    (double)rb[s][ks + 1], acc1, 0, 0, 0);
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) S.xr[4 * r + qd][16 * (2 * wave + s) + ln] = acc0[r] + acc1[r];
    }
  } else {
#pragma unroll
    for (int s = 0; s < 2; ++s)
#pragma unroll
      for (int r = 0; r < 4; ++r)
        S.xr[4 * r + qd][16 * (2 * wave + s) + ln] = (double)bf16_to_f32(S.xraw[4 * r + qd][16 * (2 * wave + s) + ln]);
  }
  __syncthreads();
  // 16 / NG threads per (token, group), 8 channels each
  constexpr int kTpg = 16 / NG;
  const int tid = wave * 64 + lane;
  const int pair = tid / kTpg, sub = tid % kTpg;
  const int t = pair / NG, gm = pair % NG;
  const int j0 = gm * G + 8 * sub;
  double v[8];
  double mn = 0.0, mx = 0.0;
  bool nan = false;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    double x = S.xr[t][j0 + e];
    x = (x < -tau) ? -tau : ((x > tau) ? tau : x);
    v[e] = x;
    nan |= (x != x);
    mn = e == 0 ? x : (x < mn ? x : mn);
    mx = e == 0 ? x : (x > mx ? x : mx);
  }
#pragma unroll
  for (int off = 1; off < kTpg; off <<= 1) {
    const double omn = __shfl_xor(mn, off), omx = __shfl_xor(mx, off);
    mn = omn < mn ? omn : mn;
    mx = omx > mx ? omx : mx;
    nan |= __shfl_xor((int)nan, off) != 0;
  }
  uint32_t sz;
  if (nan) {
    sz = nan_sz<MB>();
#pragma unroll
    for (int e = 0; e < 8; ++e) S.codes[0][t][j0 + e] = 0;
  } else {
    double sd, zd;
    sz = encode_sz<MB>((mx - mn) / 3.0, mn, sd, zd);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      double c = 0.0;
      if (sd != 0.0) {
        c = __builtin_rint((v[e] - zd) / sd);
        c = c < 0.0 ? 0.0 : (c > 3.0 ? 3.0 : c);
      }
      S.codes[0][t][j0 + e] = (uint8_t)c;
    }
  }
  if (sub == 0) S.szs[t][gm] = sz;
}

// ---- stores of one tile from LDS (wavefront 0; the exact path) ----
template <int NG, int MB>
__device__ void store_tile(Smem& S, const int32_t* dst, uint8_t* pages, int64_t n_kv, int kv, int isv, int lane) {
  constexpr Int2Layout L{NG, MB};
  const int64_t blk_bytes = L.bytes();
  // scale / zero: (t, gamma) pairs
  if (lane < 16 * NG) {
    const int t = lane / NG, gm = lane % NG;
    if (dst[t] >= 0) {
      const int64_t page = dst[t] / kPage;
      const int slot = dst[t] % kPage;
      uint8_t* blk = pages + (page * n_kv + kv) * blk_bytes;
      const int idx = isv ? (gm * kPage + slot) : (slot * NG + gm);  // V group-major, K token-major
      store_sz<MB>(blk + (isv ? L.v_sz() : L.k_sz()) + idx * MB, S.szs[t][gm]);
    }
  }
  if (!isv) {
    // K codes: lane -> (token lane/4, quarter lane%4: bytes 8*(lane%4) .. +7);
    // bits 2e of word w hold field e%4 of byte e/4
    const int t = lane >> 2, part = lane & 3;
    if (dst[t] >= 0) {
      const int64_t page = dst[t] / kPage;
      const int slot = dst[t] % kPage;
      uint8_t* blk = pages + (page * n_kv + kv) * blk_bytes;
      uint32_t w[2] = {0u, 0u};
#pragma unroll
      for (int wi = 0; wi < 2; ++wi)
#pragma unroll
        for (int e = 0; e < 16; ++e)
          w[wi] |= (uint32_t)S.codes[0][t][k_code_channel<NG>(part, wi, e >> 2, e & 3)] << (2 * e);
      *(uint2*)(blk + L.k_codes() + slot * 32 + 8 * part) = make_uint2(w[0], w[1]);
    }
  } else {
    // V codes: lane -> dword jd (channels 4jd..4jd+3) for the tokens of half th
    // of the 16; runs of tokens sharing a (page, quad) merge into one word.
    const int jd = lane & 31, th = lane >> 5;
    int64_t key = -1;
    uint32_t mask = 0u, bits = 0u;
    auto flush = [&](int64_t k, uint32_t msk, uint32_t bts) {
      if (k < 0 || msk == 0u) return;
      const int64_t page = k >> 2;
      const int q = (int)(k & 3);
      uint8_t* blk = pages + (page * n_kv + kv) * blk_bytes;
      uint32_t* word = (uint32_t*)(blk + L.v_codes() + q * kHeadDim + 4 * jd);
      if (msk == 0xffffffffu) {
        *word = bts;
      } else {
        atomicAnd(word, ~msk);
        atomicOr(word, bts);
      }
    };
    for (int t = 8 * th; t < 8 * th + 8; ++t) {
      const int32_t sl = dst[t];
      if (sl < 0) continue;
      const int64_t k = (int64_t)(sl / kPage) * 4 + ((sl % kPage) >> 2);
      if (k != key) {
        flush(key, mask, bits);
        key = k;
        mask = 0u;
        bits = 0u;
      }
      const int i = sl & 3;
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        mask |= 3u << (8 * c + 2 * i);
        bits |= (uint32_t)S.codes[0][t][4 * jd + c] << (8 * c + 2 * i);
      }
    }
    flush(key, mask, bits);
  }
}

// ---- stores of a certified tile, by every wavefront ----
// Lane (token ln, quad qd) of wavefront w holds cw[s]: the codes of channels
// 16(2w+s) + 4qd + 0..3, one per byte.  Scale/zero: the wavefront's own group.
// V: the word of a token quad is the same dword of 4 consecutive lanes, joined
// in registers (a quad broadcast), stored whole when the quad's slots are one
// aligned run, else merged token by token with atomic and/or.  K: a word takes
// dwords of two wavefronts, so it is packed from the codes in LDS (4 aligned
// dword reads), wavefront w packing tokens 4w..4w+3.  Slots: sl of token ln,
// d4 of tokens 4(ln/4) .. +3, sk of token 4w + lane/8.
template <int NG, int MB>
__device__ __forceinline__ void store_fast(const uint8_t (*codes)[kCodeRow], int32_t sl, int4 d4, int32_t sk,
                                           const uint32_t cw[2], uint32_t sz, uint8_t* pages, int64_t n_kv, int kv,
                                           int isv, int lane, int wave) {
  constexpr Int2Layout L{NG, MB};
  const int64_t blk_bytes = L.bytes();
  const int ln = lane & 15, qd = lane >> 4;
  auto block = [&](int32_t slot) { return pages + ((int64_t)(slot / kPage) * n_kv + kv) * blk_bytes; };
  if (qd == 0 && (NG == 4 || (wave & 1) == 0) && sl >= 0) {
    const int gm = NG == 4 ? wave : (wave >> 1), slot = sl % kPage;
    store_sz<MB>(block(sl) + (isv ? L.v_sz() + (gm * kPage + slot) * MB : L.k_sz() + (slot * NG + gm) * MB), sz);
  }
  if (isv) {
    const int i4 = ln & 3;
    const bool whole = d4.x >= 0 && (d4.x & 3) == 0 && d4.y == d4.x + 1 && d4.z == d4.x + 2 && d4.w == d4.x + 3;
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      const int jd = 4 * (2 * wave + s) + qd;  // dword of channels 4jd .. 4jd+3
      if (whole) {
        const uint32_t v0 = (uint32_t)__builtin_amdgcn_mov_dpp((int)cw[s], 0x00, 0xf, 0xf, false);
        const uint32_t v1 = (uint32_t)__builtin_amdgcn_mov_dpp((int)cw[s], 0x55, 0xf, 0xf, false);
        const uint32_t v2 = (uint32_t)__builtin_amdgcn_mov_dpp((int)cw[s], 0xaa, 0xf, 0xf, false);
        const uint32_t v3 = (uint32_t)__builtin_amdgcn_mov_dpp((int)cw[s], 0xff, 0xf, 0xf, false);
        if (i4 == 0)
          *(uint32_t*)(block(d4.x) + L.v_codes() + ((d4.x % kPage) >> 2) * kHeadDim + 4 * jd) =
              v0 | (v1 << 2) | (v2 << 4) | (v3 << 6);
      } else if (sl >= 0) {
        uint32_t* word = (uint32_t*)(block(sl) + L.v_codes() + ((sl % kPage) >> 2) * kHeadDim + 4 * jd);
        const int sh = 2 * (sl & 3);
        atomicAnd(word, ~(0x03030303u << sh));
        atomicOr(word, cw[s] << sh);
      }
    }
  } else if (lane < 32 && sk >= 0) {
    const int t = 4 * wave + (lane >> 3), a = (lane >> 1) & 3, w = lane & 1;
    uint32_t word = 0u;
#pragma unroll
    for (int m = 0; m < 4; ++m) word |= *(const uint32_t*)&codes[t][k_code_channel<NG>(a, w, 0, m)] << (2 * m);
    *(uint32_t*)(block(sk) + L.k_codes() + (sk % kPage) * 32 + 8 * a + 4 * w) = word;
  }
}

// The inputs of one tile for thread (token tt, channels 8cc .. 8cc+7): the
// token's INT2 slot and 8 bf16, zero and invalid for a token past `tile_end`
// or the input.  Loads are unconditional (clamped in bounds), so that the tile
// loop has no branches around them.
struct TileIn {
  int32_t slot;
  uint4 x;
  bool valid;
};
template <int MODE>
__device__ __forceinline__ TileIn fetch_tile(const QuantParams& p, const uint16_t* src, int kv, int isv, int64_t tile,
                                             int64_t tile_end, int tt, int cc) {
  TileIn in;
  const int64_t tok = tile * kTok + tt;
  in.valid = tile < tile_end && tok < p.n;
  const int64_t tc = in.valid ? tok : 0;
  in.slot = p.dst_slots[tc];
  if constexpr (MODE == 0) {
    in.x = *(const uint4*)(src + (tc * p.n_kv + kv) * kHeadDim + 8 * cc);
  } else {
    const int32_t ss = p.src_slots[tc];
    const int64_t page = ss / kPage;
    const bool ok = ss >= 0 && page < p.n_bf16_pages;
    in.valid = in.valid && ok;
    const int64_t pc = ok ? page : 0;
    const int slot = ok ? ss % kPage : 0;
    const uint16_t* blk = (const uint16_t*)(p.bf16_pages + (pc * p.n_kv + kv) * (int64_t)kBf16BlockBytes);
    if (!isv) {
      in.x = *(const uint4*)(blk + slot * kHeadDim + 8 * cc);
    } else {
      uint32_t w4[4];
#pragma unroll
      for (int e = 0; e < 4; ++e)
        w4[e] = (uint32_t)blk[kPage * kHeadDim + (8 * cc + 2 * e) * kPage + slot] |
                ((uint32_t)blk[kPage * kHeadDim + (8 * cc + 2 * e + 1) * kPage + slot] << 16);
      in.x = make_uint4(w4[0], w4[1], w4[2], w4[3]);
    }
  }
  return in;
}
// the slot a token's codes go to: -1 without a slot or past the INT2 pages
__device__ __forceinline__ int32_t tile_dst(const QuantParams& p, const TileIn& in) {
  const int32_t d = in.valid ? in.slot : -1;
  return (d >= 0 && (int64_t)(d / kPage) < p.n_int2_pages) ? d : -1;
}

// One tile per work group straight on the exact path (fp64 MFMA rotation and
// fp64 quantiser): for launches of a few tiles per matrix, where setting up
// the integer digits of R would cost more than the tiles themselves.
template <int MODE, int NG, int MB>
__global__ __launch_bounds__(kThreads) void quant_write_direct(QuantParams p) {
  extern __shared__ __align__(16) uint8_t smem_raw[];
  Smem& S = *reinterpret_cast<Smem*>(smem_raw);
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int64_t tile = blockIdx.x;
  const int kv = blockIdx.y;
  const int isv = blockIdx.z;
  const float* Rm = isv ? p.r_v : p.r_k;
  const float* R = Rm ? Rm + (int64_t)kv * kHeadDim * kHeadDim : nullptr;
  const double tau = isv ? p.tau_v : p.tau_k;
  const int tt = tid >> 4, cc = tid & 15;
  const uint16_t* src = MODE == 0 ? (isv ? p.v_src : p.k_src) : nullptr;
  float rb[2][kHeadDim / 4];
  exact_load_r(R, lane, wave, rb);  // in flight with the inputs
  const TileIn in = fetch_tile<MODE>(p, src, kv, isv, tile, tile + 1, tt, cc);
  const int32_t dslot = tile_dst(p, in);
  *(uint4*)&S.xraw[tt][8 * cc] = dslot >= 0 ? in.x : make_uint4(0u, 0u, 0u, 0u);
  if (cc == 0) S.dst_x[tt] = dslot;
  __syncthreads();
  exact_tile<NG, MB>(S, R, rb, tau, lane, wave);
  __syncthreads();
  if (wave == 0) store_tile<NG, MB>(S, S.dst_x, p.int2_pages, p.n_kv, kv, isv, lane);
}

// Digit pairs (a = x digit, b = R digit) by weight class w = a + b - 1.
#define OSCAR_PAIRS(X)                                                                                        \
  X(0, 1, 0) X(1, 0, 0) X(0, 2, 1) X(1, 1, 1) X(2, 0, 1) X(0, 3, 2) X(1, 2, 2) X(2, 1, 2) X(3, 0, 2) X(1, 3, 3) \
      X(2, 2, 3) X(3, 1, 3) X(2, 3, 4) X(3, 2, 4) X(3, 3, 5)
// the residual digit of R against the top X digit: weight 2^24 2^-38 = 256^2 2^-30, class 1

// ---- R's integer digits (A operands of the digit MFMAs) ----
// Lane l of wavefront w holds output channel 16(2w + s) + l%16; its 16 bytes
// of K half h are input channels 64h + 16(l/16) + 0..15 (the x digits use the
// same map).  Y = rint(R 2^30) as four balanced base-256 digits (ra[s][h][b],
// b = 0 the lowest), the residual lo = rint((R - Y 2^-30) 2^38) as one more
// digit (rlo[s][h]), and per lane the column terms of the error bound.  R
// null: the identity (V arriving rotated).
struct RBoundPart {
  float d1[2], d2[2], l1[2], rmax;
  bool bad;  // an entry non-finite or outside [-1.5, 1.5]
};

// store_lo(s, h, k4, word): the residual digits of four input channels, as
// soon as they are formed (the write kernel puts them straight into LDS).
template <class StoreLo>
__device__ __forceinline__ void r_digits(const float* R, int lane, int wave, u32x4 (&ra)[2][2][4], StoreLo store_lo,
                                         RBoundPart& part) {
  const int ln = lane & 15, qd = lane >> 4;
  part = RBoundPart{{0.f, 0.f}, {0.f, 0.f}, {0.f, 0.f}, 0.f, false};
  float rv[2][2][4][4];  // R[64h + 16qd + 4k4 + e][16(2w+s) + l%16], all loads in flight together
  if (R) {
#pragma unroll
    for (int s = 0; s < 2; ++s)
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int k4 = 0; k4 < 4; ++k4)
#pragma unroll
          for (int e = 0; e < 4; ++e)
            rv[s][h][k4][e] = R[(64 * h + 16 * qd + 4 * k4 + e) * kHeadDim + 16 * (2 * wave + s) + ln];
  } else {
#pragma unroll
    for (int s = 0; s < 2; ++s)
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int k4 = 0; k4 < 4; ++k4)
#pragma unroll
          for (int e = 0; e < 4; ++e)
            rv[s][h][k4][e] = (64 * h + 16 * qd + 4 * k4 + e) == 16 * (2 * wave + s) + ln ? 1.0f : 0.0f;
  }
#pragma unroll
  for (int s = 0; s < 2; ++s) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
#pragma unroll
      for (int k4 = 0; k4 < 4; ++k4) {
        uint32_t dgt[4], lo4 = 0u;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float r0 = rv[s][h][k4][e];
          const bool ok = __builtin_fabsf(r0) <= 1.5f;  // false for NaN and infinities
          part.bad |= !ok;
          const float r = ok ? r0 : 0.0f;
          const float ys = __builtin_rintf(r * 1073741824.0f);  // R 2^30, exact scaling
          // R - Y 2^-30 is exact in fp32 (both on a grid at most 24 bits below |R - Y 2^-30| <= 2^-31)
          const float dr = r - ys * 0x1p-30f;
          const float lf = __builtin_fminf(__builtin_fmaxf(__builtin_rintf(dr * 0x1p38f), -127.f), 127.f);
          part.d1[s] += __builtin_fabsf(dr);
          part.d2[s] += __builtin_fabsf(dr - lf * 0x1p-38f);
          part.l1[s] += __builtin_fabsf(r);
          part.rmax = __builtin_fmaxf(part.rmax, __builtin_fabsf(r));
          const int y = (int)ys;  // |y| <= 1.5 2^30
          dgt[e] = (uint32_t)(y + 0x808080) ^ 0x808080u;  // bytes: balanced digits e0, e1, e2 and the top digit
          lo4 |= ((uint32_t)(int)lf & 0xffu) << (8 * e);
        }
        uint32_t b0, b1;
        gather_bytes01(dgt[0], dgt[1], dgt[2], dgt[3], b0, b1);
        const uint32_t q01 = __builtin_amdgcn_perm(dgt[1], dgt[0], 0x07030602u);
        const uint32_t q23 = __builtin_amdgcn_perm(dgt[3], dgt[2], 0x07030602u);
        ra[s][h][0][k4] = b0;
        ra[s][h][1][k4] = b1;
        ra[s][h][2][k4] = __builtin_amdgcn_perm(q23, q01, 0x05040100u);
        ra[s][h][3][k4] = __builtin_amdgcn_perm(q23, q01, 0x07060302u);
        store_lo(s, h, k4, lo4);
      }
    }
  }
}

// The bound's terms over the whole matrix: column sums over the four lane
// quads, then maxima over the work group into rbits[0..3] (float bits of
// max_j sum_i |R_ij - Y_ij 2^-30|, max_j sum_i |R_ij - Y_ij 2^-30 - lo_ij
// 2^-38|, max_j sum_i |R_ij|, max |R_ij|) and bad.  rbits and bad are LDS,
// cleared and behind a barrier before the call.
__device__ __forceinline__ void r_bound_reduce(RBoundPart part, int lane, uint32_t* rbits, uint32_t* bad) {
#pragma unroll
  for (int s = 0; s < 2; ++s) {
    part.d1[s] += __shfl_xor(part.d1[s], 16);
    part.d1[s] += __shfl_xor(part.d1[s], 32);
    part.d2[s] += __shfl_xor(part.d2[s], 16);
    part.d2[s] += __shfl_xor(part.d2[s], 32);
    part.l1[s] += __shfl_xor(part.l1[s], 16);
    part.l1[s] += __shfl_xor(part.l1[s], 32);
  }
  if (part.bad) atomicOr(bad, 1u);
  if ((lane >> 4) == 0) {
    // non-negative floats order as their bit patterns
    atomicMax(&rbits[0], __builtin_bit_cast(uint32_t, __builtin_fmaxf(part.d1[0], part.d1[1])));
    atomicMax(&rbits[1], __builtin_bit_cast(uint32_t, __builtin_fmaxf(part.d2[0], part.d2[1])));
    atomicMax(&rbits[2], __builtin_bit_cast(uint32_t, __builtin_fmaxf(part.l1[0], part.l1[1])));
  }
  atomicMax(&rbits[3], __builtin_bit_cast(uint32_t, part.rmax));
}

// Prepared digits of one matrix (kRPrepBytes): ra as u32x4 [wave][s][h][b][lane],
// then rlo as u32x4 [wave][s][h][lane], then rbits[4] and bad (5 words).
__device__ __forceinline__ int r_prep_ra_index(int wave, int s, int h, int b, int lane) {
  return (((wave * 2 + s) * 2 + h) * 4 + b) * 64 + lane;
}
__device__ __forceinline__ int r_prep_lo_index(int wave, int s, int h, int lane) {
  return ((wave * 2 + s) * 2 + h) * 64 + lane;
}

// One work group per (KV head, K or V): the prepared digits of that matrix.
__global__ __launch_bounds__(kThreads) void prepare_r_kernel(const float* r_k, const float* r_v, uint8_t* prep) {
  __shared__ uint32_t rbits[4], bad;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int kv = blockIdx.x, isv = blockIdx.y;
  const float* Rm = isv ? r_v : r_k;
  const float* R = Rm ? Rm + (int64_t)kv * kHeadDim * kHeadDim : nullptr;
  if (tid < 5) (tid < 4 ? rbits[tid] : bad) = 0u;
  u32x4 ra[2][2][4], rlo[2][2];
  RBoundPart part;
  r_digits(R, lane, wave, ra, [&](int s, int h, int k4, uint32_t w) { rlo[s][h][k4] = w; }, part);
  uint8_t* base = prep + (int64_t)(kv * 2 + isv) * kRPrepBytes;
  u32x4* g_ra = (u32x4*)base;
  u32x4* g_lo = (u32x4*)(base + kRPrepRaBytes);
#pragma unroll
  for (int s = 0; s < 2; ++s)
#pragma unroll
    for (int h = 0; h < 2; ++h) {
#pragma unroll
      for (int b = 0; b < 4; ++b) g_ra[r_prep_ra_index(wave, s, h, b, lane)] = ra[s][h][b];
      g_lo[r_prep_lo_index(wave, s, h, lane)] = rlo[s][h];
    }
  __syncthreads();  // flags cleared
  r_bound_reduce(part, lane, rbits, &bad);
  __syncthreads();
  // the five words, then zeros to the end of the 256-byte tail
  if (tid < 64) ((uint32_t*)(base + kRPrepRaBytes + kRPrepLoBytes))[tid] = tid < 4 ? rbits[tid] : (tid == 4 ? bad : 0u);
}

// PREP: R's digits come prepared (p.r_prep); a separate instantiation, so the
// one that derives them keeps its own register allocation.
template <int MODE, int NG, int MB, bool PREP>
__global__ __launch_bounds__(kThreads, 2) void quant_write_kernel(QuantParams p, int tiles_per_wg) {
  extern __shared__ __align__(16) uint8_t smem_raw[];
  Smem& S = *reinterpret_cast<Smem*>(smem_raw);
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int kv = blockIdx.y;
  const int isv = blockIdx.z;
  const int64_t n_tiles = (p.n + kTok - 1) / kTok;
  const int64_t tile0 = (int64_t)blockIdx.x * tiles_per_wg;
  const int64_t tile1 = tile0 + tiles_per_wg < n_tiles ? tile0 + tiles_per_wg : n_tiles;
  if (tile0 >= tile1) return;
  const int count = (int)(tile1 - tile0);  // <= kMaxTilesPerWg
  const float* Rm = isv ? p.r_v : p.r_k;  // null: V arrives rotated (R_V folded into its projection)
  const float* R = Rm ? Rm + (int64_t)kv * kHeadDim * kHeadDim : nullptr;
  const double tau = isv ? p.tau_v : p.tau_k;
  const int ln = lane & 15, qd = lane >> 4;

  // per-thread role in the loads: token tt, channels 8cc .. 8cc+7
  const int tt = tid >> 4, cc = tid & 15;
  const uint16_t* src = MODE == 0 ? (isv ? p.v_src : p.k_src) : nullptr;
  auto fetch = [&](int64_t tile) { return fetch_tile<MODE>(p, src, kv, isv, tile, tile1, tt, cc); };
  auto dst_of = [&](const TileIn& in) { return tile_dst(p, in); };
  TileIn nx = fetch(tile0);

  // ---- set-up: this wavefront's R digits in registers (A operands), the
  // residual digit in LDS, the bound's terms over the matrix: prepared once
  // per layer (oscar_layer_prepare), or computed here ----
  u32x4 ra[2][2][4];  // [tile s][half h][digit b]
  if constexpr (PREP) {
    const uint8_t* base = p.r_prep + (int64_t)(kv * 2 + isv) * kRPrepBytes;
    const u32x4* g_ra = (const u32x4*)base;
    const u32x4* g_lo = (const u32x4*)(base + kRPrepRaBytes);
    const uint32_t* g_c = (const uint32_t*)(base + kRPrepRaBytes + kRPrepLoBytes);
#pragma unroll
    for (int s = 0; s < 2; ++s)
#pragma unroll
      for (int h = 0; h < 2; ++h) {
#pragma unroll
        for (int b = 0; b < 4; ++b) ra[s][h][b] = g_ra[r_prep_ra_index(wave, s, h, b, lane)];
        S.rlo[wave][s][h][lane] = g_lo[r_prep_lo_index(wave, s, h, lane)];
      }
    if (tid < 5) (tid < 4 ? S.rbits[tid] : S.bad_r) = g_c[tid];
    __syncthreads();
  } else {
    if (tid < 5) (tid < 4 ? S.rbits[tid] : S.bad_r) = 0u;
    RBoundPart part;
    r_digits(R, lane, wave, ra, [&](int s, int h, int k4, uint32_t w) { S.rlo[wave][s][h][lane][k4] = w; }, part);
    __syncthreads();  // flags cleared
    r_bound_reduce(part, lane, S.rbits, &S.bad_r);
    __syncthreads();
  }
  const bool bad_r = S.bad_r != 0u;
  // per-token bound = 2^E (ka + n_rounded kbr + sum |D0| kOmit), with
  // |X - 2^24 D3| <= 128 (1 + 256 + 65536) = 8421504, and 2^-44 >= 2^-45 +
  // 2^-52 for a reference's sum and the fp64 join; the float sums of at most
  // 128 terms are within 2^-17 of exact, covered by 2^-10
  const double ka = (8421504.0 * 0x1p-28 * (double)__builtin_bit_cast(float, S.rbits[0]) +
                     2.0 * (double)__builtin_bit_cast(float, S.rbits[1]) +
                     0x1p-44 * (double)__builtin_bit_cast(float, S.rbits[2])) *
                    (1.0 + 0x1p-10);
  const double kbr = 0x1p-29 * (double)__builtin_bit_cast(float, S.rbits[3]);

  // ---- stage: a tile's digits, per-token info and slots to LDS buffers ----
  auto stage = [&](int k, const TileIn& in) {
    const int32_t dslot = dst_of(in);
    const uint32_t wv[4] = {dslot >= 0 ? in.x.x : 0u, dslot >= 0 ? in.x.y : 0u, dslot >= 0 ? in.x.z : 0u,
                            dslot >= 0 ? in.x.w : 0u};  // 8 bf16 (pairs)
    S.dst[k % 3][tt] = dslot;  // the token's 16 threads write the same value
    // max |x| of the token (its 16 threads are one lane row)
    uint32_t amax = 0u;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const uint32_t a0 = wv[e] & 0x7fffu, a1 = (wv[e] >> 16) & 0x7fffu;
      amax = a0 > amax ? a0 : amax;
      amax = a1 > amax ? a1 : amax;
    }
    amax = row_max_u32(amax);
    const int efield = (int)(amax >> 7);  // bf16 exponent field of max|x|
    // exact path: non-finite (255) or tiny scale
    const bool tok_exact = dslot >= 0 && amax != 0u && (efield >= 255 || efield < 40);
    const int E = (amax == 0u || tok_exact) ? 0 : efield - 127;
    const float sc = __builtin_bit_cast(float, (uint32_t)(155 - E) << 23);  // 2^(28-E)
    uint32_t xd[8];
    int inexact = 0;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float x = bf16_to_f32((wv[e >> 1] >> (16 * (e & 1))) & 0xffffu);
      const float z = tok_exact ? 0.f : x * sc;  // |z| < 2^29
      const float zr = __builtin_rintf(z);
      inexact += zr != z ? 1 : 0;
      xd[e] = (uint32_t)((int)zr + 0x808080) ^ 0x808080u;  // balanced digits, top digit in [-32, 32]
    }
    // digit dwords of 4 channels each
    uint32_t dg[4][2];
    int dsum = 0;  // sum over the thread's channels of |D0|
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {
      const int e0 = 4 * hf;
      gather_bytes01(xd[e0], xd[e0 + 1], xd[e0 + 2], xd[e0 + 3], dg[0][hf], dg[1][hf]);
      const uint32_t q01 = __builtin_amdgcn_perm(xd[e0 + 1], xd[e0], 0x07030602u);
      const uint32_t q23 = __builtin_amdgcn_perm(xd[e0 + 3], xd[e0 + 2], 0x07030602u);
      dg[2][hf] = __builtin_amdgcn_perm(q23, q01, 0x05040100u);
      dg[3][hf] = __builtin_amdgcn_perm(q23, q01, 0x07060302u);
      dsum = (int)__builtin_amdgcn_sad_u8(dg[0][hf] ^ 0x80808080u, 0x80808080u, (uint32_t)dsum);
    }
    {
      // channel i = 8cc + e: K half i / 64, lane quad (i % 64) / 16, byte i % 16
      const int h = cc >> 3, q = (cc & 7) >> 1, off = 8 * (cc & 1);
#pragma unroll
      for (int a = 0; a < 4; ++a) *(uint2*)&S.xdig[k & 1][a][h][q][tt][off] = make_uint2(dg[a][0], dg[a][1]);
    }
    // per-token totals: sum |D0| (< 2^16) and the rounded entries
    const int tot = row_sum_i32(dsum + (inexact << 16));
    TokInfo ti;
    ti.c8 = __builtin_ldexp(1.0, E - 50);
    // an all-zero token is exactly zero
    ti.bound = amax == 0u ? 0.0 : __builtin_ldexp(ka + (double)(tot >> 16) * kbr + (double)(tot & 0xffff) * kOmit, E);
    ti.exact = tok_exact ? 1 : 0;
    ti.pad[0] = ti.pad[1] = ti.pad[2] = 0;
    S.tok[k % 3][tt] = ti;  // the token's 16 threads write the same value
  };

  // ---- digit-pair MFMAs of a staged tile: wavefront w, column tiles s = 0, 1 ----
  i32x4 acc[2][kClasses];
  auto rotate = [&](int k) {
#pragma unroll
    for (int s = 0; s < 2; ++s)
#pragma unroll
      for (int c = 0; c < kClasses; ++c) acc[s][c] = i32x4{0, 0, 0, 0};
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      u32x4 xb[4];
#pragma unroll
      for (int a = 0; a < 4; ++a) xb[a] = *(const u32x4*)&S.xdig[k & 1][a][h][qd][ln][0];
#define OSCAR_MFMA(A, B, C)                                   \
  acc[0][C] = mfma_i8(ra[0][h][B], xb[A], acc[0][C]); \
  acc[1][C] = mfma_i8(ra[1][h][B], xb[A], acc[1][C]);
      OSCAR_PAIRS(OSCAR_MFMA)
#undef OSCAR_MFMA
      acc[0][1] = mfma_i8(S.rlo[wave][0][h][lane], xb[3], acc[0][1]);
      acc[1][1] = mfma_i8(S.rlo[wave][1][h][lane], xb[3], acc[1][1]);
    }
  };

  // ---- prologue: tiles 0 and 1 staged, tile 0 rotated ----
  if (tid == 0) S.fb_n = 0u;
  {
    const TileIn in0 = nx;
    nx = fetch(tile0 + 1);
    stage(0, in0);
    const TileIn in1 = nx;
    nx = fetch(tile0 + 2);
    stage(1, in1);
  }
  __syncthreads();
  rotate(0);
  __syncthreads();  // every wavefront has read tile 0's digits before tile 2 replaces them

  for (int k = 0; k < count; ++k) {
    // ---- A: this tile's per-token info and slots, and its rotated values ----
    const TokInfo ti = S.tok[k % 3][ln];
    const int32_t* dk3 = S.dst[k % 3];
    const int32_t sl = dk3[ln];
    const int4 d4 = *(const int4*)&dk3[ln & ~3];
    const int32_t sk = dk3[4 * wave + ((lane >> 3) & 3)];
    // sum_w acc_w 256^w in the unit c8 of the lowest class:
    // (acc5 256 + acc4) 2^32 + (acc3 256 + acc2) 2^16 + (acc1 256 + acc0),
    // each term an int32 (|.| < 2^26.7, 2^30.1, 2^30.8); the inner fma is
    // exact (< 2^47), the outer one rounds once
    double xw[8];
#pragma unroll
    for (int s = 0; s < 2; ++s)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int hi = acc[s][5][r] * 256 + acc[s][4][r];
        const int mid = acc[s][3][r] * 256 + acc[s][2][r];
        const int lo = acc[s][1][r] * 256 + acc[s][0][r];
        xw[4 * s + r] = __builtin_fma((double)hi, 0x1p32, __builtin_fma((double)mid, 0x1p16, (double)lo));
      }
    // ---- B: the next tile's MFMAs run under this tile's epilogue and the staging ----
    rotate(k + 1);

    // ---- C: epilogue: lane (token ln, quad qd), channels 16(2w+s) + 4qd + r ----
    double mn = xw[0], mx = xw[0];
#pragma unroll
    for (int e = 1; e < 8; ++e) {
      mn = __builtin_fmin(mn, xw[e]);
      mx = __builtin_fmax(mx, xw[e]);
    }
    rows_minmax(mn, mx);  // the four lane rows hold the wavefront's 32 channels of the token
    if constexpr (NG == 2) {
      if (qd == 0) {
        S.part[ln][wave][0] = mn;
        S.part[ln][wave][1] = mx;
      }
      __syncthreads();
      mn = __builtin_fmin(mn, S.part[ln][wave ^ 1][0]);
      mx = __builtin_fmax(mx, S.part[ln][wave ^ 1][1]);
    }
    const double c8 = ti.c8;
    mn *= c8;  // powers of two: exact
    mx *= c8;
    // intervals holding the exact clipped min and max (and a reference's):
    // the entry bound, plus 2^-48 relative for the roundings of these steps
    const double eb = ti.bound;
    const double emn = __builtin_fma(__builtin_fabs(mn) + eb, 0x1p-48, eb);
    const double emx = __builtin_fma(__builtin_fabs(mx) + eb, 0x1p-48, eb);
    const double mn_lo = __builtin_fmin(__builtin_fmax(mn - emn, -tau), tau);
    const double mn_hi = __builtin_fmin(__builtin_fmax(mn + emn, -tau), tau);
    const double mx_lo = __builtin_fmin(__builtin_fmax(mx - emx, -tau), tau);
    const double mx_hi = __builtin_fmin(__builtin_fmax(mx + emx, -tau), tau);
    // (mx - mn) / 3 with a reference's two fp64 roundings lies in [s_lo, s_hi]
    constexpr double kThird = 1.0 / 3.0;
    const double s_lo = __builtin_fmax(mx_lo - mn_hi, 0.0) * kThird * (1.0 - 0x1p-48);
    const double s_hi = (mx_hi - mn_lo) * kThird * (1.0 + 0x1p-48);
    // the four roundings, one per lane row, then shared: z at both ends, s at both ends
    uint32_t mb[4];
    rows_gather(meta_bits<MB>(qd == 0 ? mn_lo : qd == 1 ? mn_hi : qd == 2 ? s_lo : s_hi), mb);
    const uint32_t zb = mb[0], sb = mb[2];
    bool unsure = zb != mb[1] || sb != mb[3];
    const double sv = meta_value<MB>(sb), zv = meta_value<MB>(zb);
    // 1 / s: v_rcp_f64 and two Newton steps, relative error below 2^-50 (s = 0:
    // every code is 0, taken below)
    const double sd = sv != 0.0 ? sv : 1.0;
    double inv_s = __builtin_amdgcn_rcp(sd);
    inv_s = __builtin_fma(inv_s, __builtin_fma(-sd, inv_s, 1.0), inv_s);
    inv_s = __builtin_fma(inv_s, __builtin_fma(-sd, inv_s, 1.0), inv_s);
    // t = (x c8 - z) / s = x (c8 / s) - z / s; against the exact (and the
    // reference's) t: eb / s, the rounding of z / s, the error of 1 / s over
    // |t| <= 4 and the rounding of the fma
    const double ta = c8 * inv_s, tb = -zv * inv_s;
    const double m = 0.5 - (eb * inv_s * (1.0 + 0x1p-40) + __builtin_fabs(tb) * 0x1p-52 + 0x1p-46);
    // clip at +-tau, then clamp t to [0, 3]: one clamp of t (monotone steps)
    const double tlo = __builtin_fmin(__builtin_fmax(__builtin_fma(-tau, inv_s, tb), 0.0), 3.0);
    const double thi = __builtin_fmin(__builtin_fmax(__builtin_fma(tau, inv_s, tb), 0.0), 3.0);
    // ---- the tile after next staged (inputs fetched one tile earlier); its
    // independent work fills the latency of the decision chain above ----
    {
      const TileIn in = nx;
      nx = fetch(tile0 + k + 3);
      stage(k + 2, in);
    }
    uint32_t cw[2];
    bool code_unsure = false;
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      double packed = 0.0;  // c0 + 256 c1 + 65536 c2 + 2^24 c3, exact
#pragma unroll
      for (int r = 3; r >= 0; --r) {
        const double t = __builtin_fmin(__builtin_fmax(__builtin_fma(xw[4 * s + r], ta, tb), tlo), thi);
        const double c = __builtin_rint(t);
        code_unsure |= __builtin_fabs(t - c) > m;
        packed = __builtin_fma(packed, 256.0, c);
      }
      cw[s] = sv != 0.0 ? (uint32_t)packed : 0u;
    }
    unsure |= sv != 0.0 && code_unsure;
    // codes of channels 16(2w+s) + 4qd + 0..3, one byte each
#pragma unroll
    for (int s = 0; s < 2; ++s) *(uint32_t*)&S.codes[k & 1][ln][16 * (2 * wave + s) + 4 * qd] = cw[s];
    // some decision of the tile not certified (tokens without a slot are not
    // stored and do not count); every lane writes the wavefront's answer
    S.flag[k & 1][wave] = __ballot((unsure && sl >= 0) || ti.exact || bad_r) != 0 ? 1u : 0u;
    __syncthreads();
    const uint4 fl = *(const uint4*)S.flag[k & 1];
    if ((fl.x | fl.y | fl.z | fl.w) != 0u) {
      if (tid == 0) S.fb_list[S.fb_n++] = (uint16_t)k;  // redone after the loop
    } else {
      store_fast<NG, MB>(S.codes[k & 1], sl, d4, sk, cw, sb | (zb << (4 * MB)), p.int2_pages, p.n_kv, kv, isv,
                         lane, wave);
    }
  }

  // ---- the exact path for the tiles whose decisions the bound left open ----
  __syncthreads();
  const int n_fb = (int)S.fb_n;
  for (int i = 0; i < n_fb; ++i) {
    const TileIn in = fetch(tile0 + S.fb_list[i]);
    const int32_t dslot = dst_of(in);
    *(uint4*)&S.xraw[tt][8 * cc] = dslot >= 0 ? in.x : make_uint4(0u, 0u, 0u, 0u);
    if (cc == 0) S.dst_x[tt] = dslot;
    __syncthreads();
    float rb[2][kHeadDim / 4];
    exact_load_r(R, lane, wave, rb);
    exact_tile<NG, MB>(S, R, rb, tau, lane, wave);
    __syncthreads();
    if (wave == 0) store_tile<NG, MB>(S, S.dst_x, p.int2_pages, p.n_kv, kv, isv, lane);
    __syncthreads();
  }
}

// bf16 append: K row-major, V channel-major inside the bf16 block.
__global__ __launch_bounds__(64) void bf16_write_kernel(const uint16_t* k, const uint16_t* v, const int32_t* slots,
                                                        int n_kv, uint8_t* pages, int64_t n_pages) {
  const int64_t i = blockIdx.x;
  const int kv = blockIdx.y;
  const int lane = threadIdx.x;
  const int32_t sl = slots[i];
  if (sl < 0) return;
  const int64_t page = sl / kPage;
  const int slot = sl % kPage;
  if (page >= n_pages) return;
  uint16_t* blk = (uint16_t*)(pages + (page * n_kv + kv) * (int64_t)kBf16BlockBytes);
  const uint32_t kk = *(const uint32_t*)(k + (i * n_kv + kv) * kHeadDim + 2 * lane);
  const uint32_t vv = *(const uint32_t*)(v + (i * n_kv + kv) * kHeadDim + 2 * lane);
  *(uint32_t*)(blk + slot * kHeadDim + 2 * lane) = kk;
  blk[kPage * kHeadDim + (2 * lane) * kPage + slot] = (uint16_t)(vv & 0xffffu);
  blk[kPage * kHeadDim + (2 * lane + 1) * kPage + slot] = (uint16_t)(vv >> 16);
}

__global__ __launch_bounds__(256) void copy_pages_kernel(uint8_t* base, int64_t page_bytes, int64_t n_pages,
                                                         const int32_t* src, const int32_t* dst) {
  const int64_t i = blockIdx.x;
  const int32_t s = src[i], d = dst[i];
  if (s < 0 || d < 0 || s >= n_pages || d >= n_pages || s == d) return;
  const uint4* from = (const uint4*)(base + s * page_bytes);
  uint4* to = (uint4*)(base + d * page_bytes);
  for (int64_t w = threadIdx.x; w < page_bytes / 16; w += 256) to[w] = from[w];
}

// Launches of at most this many 16-token tiles per (KV head, K or V) take the
// exact path directly.
constexpr int64_t kDirectMaxTiles = 64;

// Tiles per work group: about two work groups per compute unit in one round,
// at most kMaxTilesPerWg.
int tiles_per_wg(const QuantParams& p) {
  const int64_t n_tiles = (p.n + kTok - 1) / kTok;
  const int64_t mats = 2 * (int64_t)p.n_kv;
  int64_t wg_per_mat = 512 / mats;
  if (wg_per_mat < 1) wg_per_mat = 1;
  if (wg_per_mat > n_tiles) wg_per_mat = n_tiles;
  int64_t tpw = (n_tiles + wg_per_mat - 1) / wg_per_mat;
  return (int)(tpw < kMaxTilesPerWg ? tpw : kMaxTilesPerWg);  // more work groups beyond that
}

template <int MODE, int NG, int MB>
hipError_t launch_qw_t(const QuantParams& p, hipStream_t stream) {
  const int64_t n_tiles = (p.n + kTok - 1) / kTok;
  if (n_tiles <= kDirectMaxTiles) {
    hipLaunchKernelGGL((quant_write_direct<MODE, NG, MB>), dim3((unsigned)n_tiles, (unsigned)p.n_kv, 2),
                       dim3(kThreads), sizeof(Smem), stream, p);
    return hipGetLastError();
  }
  const int tpw = tiles_per_wg(p);
  const dim3 grid((unsigned)((n_tiles + tpw - 1) / tpw), (unsigned)p.n_kv, 2);
  const size_t lds = sizeof(Smem);
  auto kern = p.r_prep ? quant_write_kernel<MODE, NG, MB, true> : quant_write_kernel<MODE, NG, MB, false>;
  hipLaunchKernelGGL(kern, grid, dim3(kThreads), lds, stream, p, tpw);
  return hipGetLastError();
}

template <int MODE>
hipError_t launch_qw(const QuantParams& p, hipStream_t stream) {
  if (p.group == 32 && p.mb == 4) return launch_qw_t<MODE, 4, 4>(p, stream);
  if (p.group == 32) return launch_qw_t<MODE, 4, 2>(p, stream);
  if (p.mb == 4) return launch_qw_t<MODE, 2, 4>(p, stream);
  return launch_qw_t<MODE, 2, 2>(p, stream);
}

}  // namespace

hipError_t launch_prepare_r(const float* r_k, const float* r_v, int n_kv, uint8_t* prep, hipStream_t stream) {
  hipLaunchKernelGGL(prepare_r_kernel, dim3((unsigned)n_kv, 2), dim3(kThreads), 0, stream, r_k, r_v, prep);
  return hipGetLastError();
}

hipError_t launch_quant_write(const QuantParams& p, int mode, hipStream_t stream) {
  if (p.n == 0) return hipSuccess;
  return mode == 0 ? launch_qw<0>(p, stream) : launch_qw<1>(p, stream);
}

hipError_t launch_bf16_write(const uint16_t* k, const uint16_t* v, const int32_t* slots, int64_t n, int n_kv,
                             uint8_t* bf16_pages, int64_t n_pages, hipStream_t stream) {
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(bf16_write_kernel, dim3((unsigned)n, (unsigned)n_kv), dim3(64), 0, stream, k, v, slots, n_kv,
                     bf16_pages, n_pages);
  return hipGetLastError();
}

hipError_t launch_copy_pages(uint8_t* base, int64_t block_bytes_all_heads, int64_t n_pages, const int32_t* src,
                             const int32_t* dst, int64_t n, hipStream_t stream) {
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(copy_pages_kernel, dim3((unsigned)n), dim3(256), 0, stream, base, block_bytes_all_heads,
                     n_pages, src, dst);
  return hipGetLastError();
}

}  // namespace oscar
