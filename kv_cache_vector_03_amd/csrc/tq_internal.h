// Internal declarations shared by the host library and the HIP kernels.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>
#include <string>
#include <vector>

#include "tq_api.h"

namespace tq {

// Per-context device tables.
struct DevTables {
  const float* centroids = nullptr;    // [2^k_bits] fp32
  const float* thresholds = nullptr;   // [2^k_bits - 1] fp32
  const float* signs1 = nullptr;       // D1 as fp32 +-1 [d]
  const float* signs2 = nullptr;       // D2 as fp32 +-1 [d]
  const float* S = nullptr;            // [d][d] fp32 row-major
  // S^T as MFMA B-operand tiles of v_mfma_f32_16x16x32_f16, fp16 hi/lo split
  // of (S * 2^kSScaleLog2): tile (nt, kt) holds lane l, element e =
  // S[16 nt + l%16][32 kt + 8 (l/16) + e]; layout [nt][kt][hi,lo][64][8] fp16.
  const uint16_t* s_tiles = nullptr;
  // The same tiles for S diag(D2) (the columns j with D2_j = -1 negated,
  // exactly: negating an fp16 hi/lo pair negates both parts).
  const uint16_t* s_tiles_d2 = nullptr;
  // Decode pair table: entry a | b << k_bits = (bf16 hi c[a], bf16 hi c[b]),
  // (bf16 lo c[a], bf16 lo c[b]) as two dwords; [2^(2 k_bits)][2] uint32
  // (2-4-bit keys only: empty for 8-bit keys).
  const uint32_t* pair_lut = nullptr;
  // One-code table (the 8-bit decode): entry a = bf16 hi c[a] | bf16 lo c[a] << 16.
  const uint32_t* code_lut = nullptr;
  // The same pair table in fp16 (extend attention): entry a | b << k_bits =
  // (fp16 hi c[a], fp16 hi c[b]), (fp16 lo c[a], fp16 lo c[b]); [2^(2 k_bits)][2].
  const uint32_t* pair_lut_f16 = nullptr;
  // S diag(D2) as MFMA A-operand tiles for the head_dim-128 store kernel whose
  // residual operand comes straight from the rotation's output registers:
  // tile (nt, kt) lane l element e = 16 S[16 nt + l % 16][j] D2[j] with
  // j = 32 kt + 16 (e / 4) + 4 (l / 16) + e % 4, fp16 hi / lo;
  // layout [nt][kt][hi, lo][64][8] fp16 (empty for head_dim 256).
  const uint16_t* s_tiles_perm_d2 = nullptr;
  // Equally spaced codebook (c_k = c0 + k step, c0 = -(L-1) step / 2): the
  // step, which the decode uses to take c[idx] arithmetically; 0 for a
  // Lloyd-Max codebook.
  float uni_step = 0.f;
};

struct Layout {
  int64_t kcodes, kqjl, kmeta, vcodes, vmeta, bytes;
};

}  // namespace tq

struct tq_ctx {
  tq_preset preset;
  int device = 0;
  int d = 0, kb = 0, vb = 0;
  bool qjl = true;   // false: MSE-only keys (no sign bits, no residual norm)
  bool rotv = false; // values rotated before their group quantisation
  std::vector<double> c64, t64;
  std::vector<float> c32, t32;
  std::vector<int8_t> signs;  // [2][d]
  std::vector<float> S;       // [d][d]
  tq::Layout lay;
  tq::DevTables dev;
  void* dev_block = nullptr;  // one allocation holding every device table
};

namespace tq {

constexpr int kSScaleLog2 = 4;   // S is pre-scaled by 16 before the fp16 split
constexpr int kRScaleLog2 = 6;   // r is pre-scaled by 64 before the fp16 split

void set_error(const char* fmt, ...);

Layout make_layout(int d, int kb, int vb, bool qjl);

// Kernel launchers (defined in the .hip files); return a hipError_t.
hipError_t launch_quantize(const tq_ctx* c, const void* k, const void* v, int in_dtype, int64_t num_tokens,
                           int num_kv_heads, const int32_t* slot_mapping, void* pool, int64_t num_blocks,
                           hipStream_t stream);

// The head_dim-128 bf16 store kernel with the rotation and the QJL projection
// on the matrix cores (tq_quantize_mfma.hip); values not rotated.
hipError_t launch_quantize_mfma(const tq_ctx* c, const void* k, const void* v, int64_t num_tokens, int num_kv_heads,
                                const int32_t* slot_mapping, void* pool, int64_t num_blocks, hipStream_t stream);

struct DecodePlan {
  int d, G, num_splits_max, chunk;
  size_t off_part, bytes;
};
DecodePlan plan_decode(const tq_decode_args* a);
hipError_t launch_decode(const tq_decode_args* a, const DecodePlan& plan, hipStream_t stream);
// Host-side check that every kernel of the decode fits a compute unit (LDS of
// the recent window beside the kernel's own tables); on failure the message is
// set with set_error and an error is returned.  Enqueues nothing.
hipError_t check_decode_launch(const tq_decode_args* a, const DecodePlan& plan);
// Extend attention (tq_extend.hip).
hipError_t launch_extend(const tq_extend_args* a, hipStream_t stream);
// Device address of the current device's static scratch array of
// TQ_NOALLOC_SCRATCH_BYTES bytes (looked up once per device, then cached).
hipError_t noalloc_scratch(void** out);

}  // namespace tq
