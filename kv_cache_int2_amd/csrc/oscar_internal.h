// Internal declarations shared by the host library and the HIP kernel files.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace oscar {

constexpr int kHeadDim = 128;
constexpr int kPage = 16;

// Byte offsets inside an INT2 (page, KV head) block; ng = head_dim / group,
// mb = bytes of one (scale, zero) pair: 4 (two fp16) or 2 (two FP8 E4M3, the
// lower-metadata format).
struct Int2Layout {
  int ng;
  int mb;
  __host__ __device__ constexpr int k_codes() const { return 0; }
  __host__ __device__ constexpr int k_sz() const { return kPage * kHeadDim / 4; }
  __host__ __device__ constexpr int v_codes() const { return k_sz() + kPage * ng * mb; }
  __host__ __device__ constexpr int v_sz() const { return v_codes() + kPage * kHeadDim / 4; }
  __host__ __device__ constexpr int bytes() const { return v_sz() + kPage * ng * mb; }
};
constexpr int kBf16BlockBytes = 4 * kPage * kHeadDim;

// K codes: a token's 32 bytes are four 8-byte quarters a (one per lane quad of
// the attention kernel), each two 32-bit words w; byte i of a word holds four
// 2-bit fields, field m at bits 2m.  This gives the channel in field m of byte
// i of word w of quarter a.  Every field position of a word belongs to one
// group, so (word >> 2m) & 0x03030303 is four int8 codes of one group:
//   32-channel groups (ng = 4): channel 64w + 32(m/2) + 8a + 4(m%2) + i
//     (fields 0, 1: group 2w; fields 2, 3: group 2w + 1);
//   64-channel groups (ng = 2): channel 64w + 16a + 4m + i (word w: group w).
template <int NG>
__host__ __device__ constexpr int k_code_channel(int a, int w, int i, int m) {
  return NG == 4 ? 64 * w + 32 * (m >> 1) + 8 * a + 4 * (m & 1) + i : 64 * w + 16 * a + 4 * m + i;
}

struct QuantParams {
  const uint16_t* k_src;      // dense bf16 [n][n_kv][d]            (mode 0)
  const uint16_t* v_src;
  const uint8_t* bf16_pages;  // bf16 storage for requantisation    (mode 1)
  int64_t n_bf16_pages;
  const int32_t* src_slots;   // bf16 physical slots                (mode 1)
  const int32_t* dst_slots;   // INT2 physical slots
  uint8_t* int2_pages;
  int64_t n_int2_pages;
  const float* r_k;           // [n_kv][d][d]
  const float* r_v;
  double tau_k, tau_v;
  int64_t n;
  int n_kv;
  int group;
  int mb;                     // bytes of a (scale, zero) pair: 4 or 2
  const uint8_t* r_prep;      // R's digits prepared per matrix (oscar_layer_prepare), or null
};

// R's digits prepared for the write kernel, per (KV head, K or V) matrix: the
// four base-256 digits as MFMA A operands (4 wavefronts x 64 lanes x 16
// u32x4), the residual digit (4 x 64 x 4 u32x4), the bound's five words,
// padded to 256 bytes.
constexpr size_t kRPrepRaBytes = size_t(4) * 2 * 2 * 4 * 64 * 16;
constexpr size_t kRPrepLoBytes = size_t(4) * 2 * 2 * 64 * 16;
constexpr size_t kRPrepBytes = kRPrepRaBytes + kRPrepLoBytes + 256;

// Step tables carried in the prologue's launch arguments: rows 0-3 the step's
// slots, row 4 the context lengths, each of kArgBatch entries.
constexpr int kArgBatch = 64;
struct ArgTables {
  int32_t v[5][kArgBatch];
};

struct DecodeParams {
  const uint8_t* int2_pages;
  int64_t n_int2_pages;
  const uint8_t* bf16_pages;
  int64_t n_bf16_pages;
  const uint16_t* q;          // bf16 [B][Hq][d]
  const float* r_k;           // [n_kv][d][d]
  const float* r_v;
  const int32_t* int2_bt;
  int max_int2_pages;
  const int32_t* bf16_bt;
  int max_bf16_pages;
  const int32_t* ctx_lens;
  // Query heads as the kernels see them: g per KV head, n_q = n_kv g.  In
  // decode these are the model's heads.  In chunked prefill they are virtual:
  // head hv of KV head kv is query chunk0 + hv / g_real of the chunk, model
  // head kv g_real + hv % g_real (q_row, q_pos).
  int batch, n_q, n_kv, g, ng, ct;
  int q_heads;                // query heads of one token in q and out (Hq)
  int g_real;                 // model query heads per KV head
  int chunk;                  // queries per request in q and out (1 in decode)
  int chunk0;                 // first of them handled by this launch
  int mb;                     // bytes of a (scale, zero) pair in the INT2 blocks: 4 or 2
  int sink, recent;           // region rule (baseline: sink huge, recent 0)
  int splits_int2, splits_bf16;
  int bf16_in_combine;        // bf16 splits (<= 4) run by the combine kernel's wavefronts
  // small grids: the bf16 splits run as extra items of the INT2 kernel's grid,
  // and the combine takes one work group per (request, KV head, query head)
  int small_grid;
  float p_scale_exp;          // P' is scaled by 2^p_scale_exp before fp16 rounding
  // workspace carve-up
  uint32_t* qb;               // [B*n_kv][ct][1536] int8x4 words: digits of 2Q as MFMA A operands
  float* qaux;                // [B*n_kv][1 + 16*ct]: logit factor, 2 Qbar per row
  float* partial;             // [B][Hq][splits][2 + d]: m (log2), l, acc
  float* out;                 // [B][Hq][d]
  // fused decode-step writes (step_slots null: none), done by the prologue
  // kernel before the attention kernels read the cache
  const int32_t* step_slots;  // [4][B]: INT2 slot and bf16 slot of the new token,
                              // bf16 source and INT2 destination of the token leaving the window
  const uint16_t* k_new;      // bf16 [B][n_kv][d]: the step's new token
  const uint16_t* v_new;
  uint8_t* int2_w;            // writable views of the two storages
  uint8_t* bf16_w;
  int split_writes;           // the writes in work groups of their own (small batches): 1 per pair, 2 per matrix
  double tau_k, tau_v;
  int has_step;               // the step's writes run (step_slots, or the argument tables)
  // oscar_decode_step_host_tables: the step's [4][B] slots and ctx_lens, given
  // in host memory, travel in the prologue's launch arguments (ArgTables, B <=
  // kArgBatch); step_slots is then null, and the prologue copies the lengths
  // to ctx_w, a workspace array that ctx_lens names for the later kernels
  int arg_tables;
  int32_t* ctx_w;
};

// How the 16-row tiles of a (request, KV head) spread over the wavefronts of
// one INT2 work item: CT tiles per wavefront (they share the unpacked codes,
// at waves_per_simd(CT) wavefronts per SIMD), W wavefronts (they share the
// staged pages).
struct TileSplit {
  int ct, w;
};
// Four tiles (at 32-channel groups: 16 heads, three real tiles padded with an
// empty fourth) go to one wide wavefront, whose value MFMAs take the 16 heads
// as rows (two wavefronts per SIMD).
inline TileSplit tile_split(int tiles) {
  switch (tiles) {
    case 2: return {2, 1};
    case 3: return {1, 3};
    case 4: return {4, 1};
    default: return {1, 1};
  }
}
// wavefronts per SIMD of a decode INT2 item whose wavefronts take ct tiles
inline int waves_per_simd(int ct) { return ct == 1 ? 4 : (ct == 2 ? 3 : 2); }

hipError_t launch_quant_write(const QuantParams& p, int mode, hipStream_t stream);
// R's digits for every (KV head, K or V) matrix into prep (n_kv 2 kRPrepBytes)
hipError_t launch_prepare_r(const float* r_k, const float* r_v, int n_kv, uint8_t* prep, hipStream_t stream);
hipError_t launch_bf16_write(const uint16_t* k, const uint16_t* v, const int32_t* slots, int64_t n, int n_kv,
                             uint8_t* bf16_pages, int64_t n_pages, hipStream_t stream);
hipError_t launch_copy_pages(uint8_t* base, int64_t block_bytes_all_heads, int64_t n_pages, const int32_t* src,
                             const int32_t* dst, int64_t n, hipStream_t stream);
// ev_start / ev_stop (may be null): recorded on `stream` around the main kernel.
hipError_t launch_decode(const DecodeParams& p, hipStream_t stream, hipEvent_t ev_start, hipEvent_t ev_stop,
                         const ArgTables* tabs = nullptr);
// One query block of a chunked prefill (p.ct = 4, 8 or 16 tiles, one wavefront each).
hipError_t launch_prefill(const DecodeParams& p, hipStream_t stream, hipEvent_t ev_start, hipEvent_t ev_stop);

// Workspace bytes for the decode path (each region 256-byte aligned).
size_t decode_workspace_bytes(int batch, int n_q, int n_kv, int ct, int splits_total);
void decode_workspace_carve(DecodeParams& p, void* ws);

// The allocation-free decode's workspace: a device array of this size in the
// library (one copy per GPU, held until the process ends).  decode_scratch
// returns its address on the device of `stream` (the current device for the
// null stream), looking the address up on the first call per device.
constexpr size_t kDecodeScratchBytes = size_t(64) << 20;
hipError_t decode_scratch(hipStream_t stream, void** ptr, size_t* bytes);

}  // namespace oscar
