// OSCAR write path for gfx950: rotate, clip, per-token asymmetric INT2 per
// channel group, pack into the paged INT2 blocks.
//
// [ES] "El sistema de servicio", write path: each token is rotated by the fixed
// calibrated rotation, clipped at the calibrated percentile threshold, and
// quantised to asymmetric INT2 per token with a group of channels sharing a
// scale and zero point.  [IT] 2.2.B: the history lives in INT2 after the fixed
// rotation and clip.
//
// One block of eight wavefronts handles 16 tokens of one KV head and one of
// K / V:  x_rot[16][128] = X[16][128] R[128][128]  on v_mfma_f64_16x16x4_f64,
// wavefront w producing columns 16w..16w+15 (its 32 values of R are loaded
// together, so the block waits for memory once); then 8 (G=32) or 16 (G=64)
// threads per (token, group) clip, reduce min/max with shuffles and code 4
// channels each.
// X holds bf16 values and R fp32 values; both are exact in fp64 and so are
// their products, and the sums are fp64.  The quantiser's decisions (fp16
// rounding of scale and zero, the code of each element) are therefore taken on
// an fp64 rotated value, the same precision a double-precision reference uses.
// Per group: mn, mx; s = fp16((mx - mn) / 3), z = fp16(mn), one rounding from
// fp64, nearest-even; code = clamp(rint((x - z) / s), 0, 3) in fp64 (IEEE
// division, rint = nearest-even).  The lower-metadata format (MB = 2) rounds s
// and z to FP8 E4M3 instead, the same way.
//
// Storage (per (page, KV head) block): K codes token-major (a token's 32 bytes
// are its own) with token-major scale/zero, V codes by token quad [4][128]
// bytes (byte j of quad q: channel j of tokens 4q..4q+3) with group-major
// scale/zero.  A V dword (4 channels of one quad) is written whole when this
// wavefront holds all 4 tokens of the quad, else merged with 32-bit atomic
// and/or, so tokens of one page may be written by different wavefronts or
// launches.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "oscar_internal.h"
#include "quant_common.h"

namespace oscar {
namespace {

typedef double f64x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __builtin_bit_cast(float, (uint32_t)b << 16); }

template <int MODE, int NG, int MB>
__global__ __launch_bounds__(512) void quant_write_kernel(QuantParams p) {
  constexpr int G = kHeadDim / NG;
  constexpr Int2Layout L{NG, MB};
  constexpr int kTpg = 32 / NG;  // threads per (token, group), 4 channels each
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int64_t t0 = (int64_t)blockIdx.x * 16;
  const int kv = blockIdx.y;
  const int isv = blockIdx.z;
  __shared__ float xin[16][kHeadDim + 1];
  __shared__ double xr[16][kHeadDim + 1];
  __shared__ uint8_t codes[16][kHeadDim];
  __shared__ uint32_t szs[16][NG];
  __shared__ int32_t dst[16];

  if (tid < 16) {
    const int64_t t = t0 + tid;
    dst[tid] = (t < p.n) ? p.dst_slots[t] : -1;
    if (dst[tid] >= 0 && (int64_t)(dst[tid] / kPage) >= p.n_int2_pages) dst[tid] = -1;
  }
  __syncthreads();
  // ---- stage inputs (bf16 values) ----
  for (int idx = tid; idx < 16 * kHeadDim; idx += 512) {
    const int t = idx / kHeadDim, j = idx % kHeadDim;
    float v = 0.f;
    if (dst[t] >= 0) {
      if constexpr (MODE == 0) {
        const uint16_t* src = isv ? p.v_src : p.k_src;
        v = bf16_to_f32(src[((t0 + t) * p.n_kv + kv) * kHeadDim + j]);
      } else {
        const int32_t ss = p.src_slots[t0 + t];
        const int64_t page = ss / kPage;
        const int slot = ss % kPage;
        if (ss >= 0 && page < p.n_bf16_pages) {
          const uint16_t* blk = (const uint16_t*)(p.bf16_pages + (page * p.n_kv + kv) * (int64_t)kBf16BlockBytes);
          v = bf16_to_f32(isv ? blk[kPage * kHeadDim + j * kPage + slot] : blk[slot * kHeadDim + j]);
        }
      }
    }
    xin[t][j] = v;
  }
  // ---- x_rot = X R in fp64 on MFMA: wavefront w owns output columns 16w..16w+15 ----
  // f64 16x16x4 operands: A lane l -> A[l%16][l/16]; B lane l -> B[l/16][l%16];
  // C lane l, element r -> C[4r + l/16][l%16].
  // (R_V null: V arrives rotated, its projection having R_V folded in)
  const float* Rm = isv ? p.r_v : p.r_k;
  const int ln = lane & 15, qd = lane >> 4;
  if (Rm) {
    const float* R = Rm + (int64_t)kv * kHeadDim * kHeadDim;
    float rb[kHeadDim / 4];  // this lane's B values, loaded together
#pragma unroll
    for (int ks = 0; ks < kHeadDim / 4; ++ks) rb[ks] = R[(4 * ks + qd) * kHeadDim + 16 * wave + ln];
    __syncthreads();
    f64x4 acc = f64x4{0.0, 0.0, 0.0, 0.0};
#pragma unroll
    for (int ks = 0; ks < kHeadDim / 4; ++ks)
      acc = __builtin_amdgcn_mfma_f64_16x16x4f64((double)xin[ln][4 * ks + qd], (double)rb[ks], acc, 0, 0, 0);
#pragma unroll
    for (int r = 0; r < 4; ++r) xr[4 * r + qd][16 * wave + ln] = acc[r];
  } else {
    __syncthreads();
    for (int idx = tid; idx < 16 * kHeadDim; idx += 512) xr[idx / kHeadDim][idx % kHeadDim] = xin[idx / kHeadDim][idx % kHeadDim];
  }
  __syncthreads();
  // ---- clip, group statistics, codes: kTpg threads per (token, group) ----
  {
    const int pair = tid / kTpg, sub = tid % kTpg;
    const int t = pair / NG, gm = pair % NG;
    const int j0 = gm * G + 4 * sub;
    const double tau = isv ? p.tau_v : p.tau_k;
    double v[4];
    double mn = 0.0, mx = 0.0;
    bool nan = false;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      double x = xr[t][j0 + e];
      x = (x < -tau) ? -tau : ((x > tau) ? tau : x);
      v[e] = x;
      nan |= (x != x);
      mn = e == 0 ? x : (x < mn ? x : mn);
      mx = e == 0 ? x : (x > mx ? x : mx);
    }
    // the kTpg threads of a (token, group) are consecutive lanes of one wavefront
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
      for (int e = 0; e < 4; ++e) codes[t][j0 + e] = 0;
    } else {
      double sd, zd;
      sz = encode_sz<MB>((mx - mn) / 3.0, mn, sd, zd);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        double c = 0.0;
        if (sd != 0.0) {
          c = __builtin_rint((v[e] - zd) / sd);
          c = c < 0.0 ? 0.0 : (c > 3.0 ? 3.0 : c);
        }
        codes[t][j0 + e] = (uint8_t)c;
      }
    }
    if (sub == 0) szs[t][gm] = sz;
  }
  __syncthreads();
  if (tid >= 64) return;
  // ---- stores ----
  uint8_t* pages = p.int2_pages;
  const int64_t blk_bytes = L.bytes();
  // scale / zero: (t, gamma) pairs
  if (lane < 16 * NG) {
    const int t = lane / NG, gm = lane % NG;
    if (dst[t] >= 0) {
      const int64_t page = dst[t] / kPage;
      const int slot = dst[t] % kPage;
      uint8_t* blk = pages + (page * p.n_kv + kv) * blk_bytes;
      const int idx = isv ? (gm * kPage + slot) : (slot * NG + gm);  // V group-major, K token-major
      store_sz<MB>(blk + (isv ? L.v_sz() : L.k_sz()) + idx * MB, szs[t][gm]);
    }
  }
  if (!isv) {
    // K codes: lane -> (token lane/4, quarter lane%4: bytes 8*(lane%4) .. +7);
    // bits 2e of word w hold field e%4 of byte e/4
    const int t = lane >> 2, part = lane & 3;
    if (dst[t] >= 0) {
      const int64_t page = dst[t] / kPage;
      const int slot = dst[t] % kPage;
      uint8_t* blk = pages + (page * p.n_kv + kv) * blk_bytes;
      uint32_t w[2] = {0u, 0u};
#pragma unroll
      for (int wi = 0; wi < 2; ++wi)
#pragma unroll
        for (int e = 0; e < 16; ++e)
          w[wi] |= (uint32_t)codes[t][k_code_channel<NG>(part, wi, e >> 2, e & 3)] << (2 * e);
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
      uint8_t* blk = pages + (page * p.n_kv + kv) * blk_bytes;
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
        bits |= (uint32_t)codes[t][4 * jd + c] << (8 * c + 2 * i);
      }
    }
    flush(key, mask, bits);
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

template <int MODE>
hipError_t launch_qw(const QuantParams& p, hipStream_t stream) {
  const dim3 grid((unsigned)((p.n + 15) / 16), (unsigned)p.n_kv, 2);
  if (p.group == 32 && p.mb == 4)
    hipLaunchKernelGGL((quant_write_kernel<MODE, 4, 4>), grid, dim3(512), 0, stream, p);
  else if (p.group == 32)
    hipLaunchKernelGGL((quant_write_kernel<MODE, 4, 2>), grid, dim3(512), 0, stream, p);
  else if (p.mb == 4)
    hipLaunchKernelGGL((quant_write_kernel<MODE, 2, 4>), grid, dim3(512), 0, stream, p);
  else
    hipLaunchKernelGGL((quant_write_kernel<MODE, 2, 2>), grid, dim3(512), 0, stream, p);
  return hipGetLastError();
}

}  // namespace

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
