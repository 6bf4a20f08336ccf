// Extend (chunked prefill) attention over the compressed paged cache plus the
// chunk's own bf16 keys and values, for gfx950 (Roadmap §4.1: a fused extend
// kernel over the compressed pool beside the fused decode kernel; §4.4: the
// prefill path is where rotation and quantisation cost shows).
//
// One workgroup of eight waves per (sequence b, KV head h, tile of 128 query
// rows); a row is one (chunk token, query head) pair, row r = token r / G,
// head h G + r % G, and wave w owns rows 16 w .. 16 w + 15.  The workgroup
// reads the compressed prefix once, 32 tokens (two paged records) per step,
// software-pipelined with one barrier per step (the records of step s + 2 are
// stored and those of step s + 3 loaded while step s + 1 is built and step s
// computed):
//   build  (all 512 threads): the step's records go to LDS, and from them the
//          MFMA B tiles every wave shares: the rotated centroids c[idx] of the
//          32 tokens as fp16 hi and lo parts (two codes per lookup of an fp16
//          pair table), the QJL sign bits as fp16 +-1 (one lookup per sign
//          byte) and the dequantised values q s + z as fp16 hi and lo parts;
//   score  (per wave) on v_mfma_f32_16x16x32_f16: 16 query rows x 16 tokens,
//          A = q~ (fp16 hi/lo, per-row power-of-two scale, log2(e) sm_scale
//          folded in), three products per k-slice (hi.hi + hi.lo + lo.hi);
//          the QJL sum likewise with A = p = S q~ and B = +-1; n_t and gamma_t
//          scale the token columns;
//   softmax online per row in the exp2 domain with a lazily moved reference
//          (as in decode); the weights go through LDS into the A layout;
//   values acc[row][channel] += P . v^, three fp16 products per tile.
// Then the chunk's own tokens, 32 keys per step, causally: K tile (bf16,
// exact products with the bf16 query) and V tile (transposed, fp16) in LDS.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <mutex>

#include "tq_common.hip.h"
#include "tq_internal.h"

namespace tq {
namespace {

typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

constexpr int ED = 128;                 // head_dim of the extend kernels
constexpr int EKT = ED / 32;            // k-slices of one MFMA row
constexpr int ENW = 8;                  // waves per workgroup
constexpr int ERPW = 16;                // query rows per wave
constexpr int EROWS = ENW * ERPW;       // query rows per workgroup
constexpr int EKR = ED + 8;             // chunk K tile row stride (bf16 elements)
constexpr int EVS = 40;                 // chunk V tile row stride (fp16 elements: 32 tokens + pad)
constexpr int EPS = 36;                 // weight staging row stride (floats)
constexpr float kELazy = 2.0f;          // lazy softmax reference margin (log2 units)

template <int KB, int VB, bool QJ>
struct ERec {  // byte layout of one (block, KV head) record, as the host lays it out
  static constexpr int kcodes = 0;
  static constexpr int kqjl = kcodes + 16 * (KB * ED / 8);
  static constexpr int kmeta = kqjl + (QJ ? 16 * (ED / 8) : 0);
  static constexpr int kmeta_slot = QJ ? 4 : 2;
  static constexpr int vcodes = kmeta + 16 * kmeta_slot;
  static constexpr int vmeta = vcodes + (VB * ED / 8) * 16;
  static constexpr int bytes = vmeta + (ED / 32) * 64;
  static constexpr int pieces = bytes / 16;
};

constexpr int align16(int x) { return (x + 15) & ~15; }

template <int KB, int VB, bool QJ>
struct ELds {
  using R = ERec<KB, VB, QJ>;
  static constexpr int pair = 0;                                  // uint2 [2^(2 KB)]
  static constexpr int sgn = pair + 8 * (1 << (2 * KB));          // u32x4 [256] (QJL)
  static constexpr int rows = sgn + (QJ ? 256 * 16 : 0);          // float uq[EROWS], up[EROWS]
  static constexpr int ring = rows + 2 * EROWS * 4;               // three slots of a step's two records
  static constexpr int ring_slot = align16(2 * R::bytes);
  static constexpr int kc = align16(ring + 3 * ring_slot);        // two buffers of u32x4 [2 half][EKT][2 part][64]
  static constexpr int kc_buf = 2 * EKT * 2 * 64 * 16;
  static constexpr int ks = kc + 2 * kc_buf;                      // two buffers of u32x4 [2 half][EKT][64]
  static constexpr int ks_buf = QJ ? 2 * EKT * 64 * 16 : 0;
  static constexpr int vt = ks + 2 * ks_buf;                      // two buffers of u32x4 [8 ct][2 part][64]
  static constexpr int vt_buf = 8 * 2 * 64 * 16;
  static constexpr int ps = vt + 2 * vt_buf;                      // float [ENW][16][EPS]
  static constexpr int ck = ps + ENW * 16 * EPS * 4;              // bf16 [32][EKR]
  static constexpr int cv = ck + 32 * EKR * 2;                    // fp16 [ED][EVS]
  static constexpr int end = cv + ED * EVS * 2;
  static constexpr int stage = kc;                                // prologue: float q~ [EROWS][ED], p [EROWS][ED]
  static constexpr int stage_end = stage + 2 * EROWS * ED * 4;
  static constexpr int total = end > stage_end ? end : stage_end;
  static_assert(total <= 160 * 1024, "extend workgroup LDS");
};

struct EArgs {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const int32_t* cu;
  int B, Hq, Hkv, G, max_chunk;
  const uint8_t* pool;
  int64_t pool_blocks, rec;
  DevTables dev;
  const int32_t* bt;
  int max_blocks;
  const int32_t* prefix_lens;
  int max_prefix;
  float logit_scale;  // sm_scale * log2(e)
  float* out;
  int qtiles;         // query tiles per (sequence, KV head)
};

__device__ __forceinline__ uint32_t pack_f16x2(float a, float b) {
  return (uint32_t)f32_to_f16_bits(a) | ((uint32_t)f32_to_f16_bits(b) << 16);
}
// fp16 hi / lo parts of x (hi = fp16(x), lo = fp16(x - hi))
__device__ __forceinline__ void split_f16(float x, _Float16& hi, _Float16& lo) {
  hi = (_Float16)x;
  lo = (_Float16)(x - (float)hi);
}
// fp16 hi / lo parts of two values packed in dwords: hi truncated (round
// toward zero, one instruction for both), x - hi exact in fp32, lo truncated:
// x = hi + lo to ~2^-22 relative
__device__ __forceinline__ uint2 split2_f16(float x, float y) {
  const auto h = __builtin_amdgcn_cvt_pkrtz(x, y);
  const auto l = __builtin_amdgcn_cvt_pkrtz(x - (float)h[0], y - (float)h[1]);
  return make_uint2(__builtin_bit_cast(uint32_t, h), __builtin_bit_cast(uint32_t, l));
}
// acc[ct][r] *= a for the eight column tiles of one output row, skipped when
// go == 0, as one block whose branch the compiler does not see: the
// accumulators stay in their registers on both paths.  Written as a C++
// branch, the compiler renames them inside it and copies all 32 of them on
// the (common) path that skips it, every step (prefill workload 1400 -> 1370
// us without those copies).  The accumulators were last written by the value
// products of the previous step, a barrier and the whole score phase earlier.
template <int CT>
__device__ __forceinline__ void rescale_row(f32x4 (&acc)[CT], int r, float a, uint32_t go) {
  static_assert(CT == 8, "eight column tiles");
  float e0 = acc[0][r], e1 = acc[1][r], e2 = acc[2][r], e3 = acc[3][r];
  float e4 = acc[4][r], e5 = acc[5][r], e6 = acc[6][r], e7 = acc[7][r];
  asm volatile(
      "s_cmp_eq_u32 %9, 0\n\t"
      "s_cbranch_scc1 .Lrs_skip%=\n\t"
      "v_mul_f32 %0, %0, %8\n\t"
      "v_mul_f32 %1, %1, %8\n\t"
      "v_mul_f32 %2, %2, %8\n\t"
      "v_mul_f32 %3, %3, %8\n\t"
      "v_mul_f32 %4, %4, %8\n\t"
      "v_mul_f32 %5, %5, %8\n\t"
      "v_mul_f32 %6, %6, %8\n\t"
      "v_mul_f32 %7, %7, %8\n"
      ".Lrs_skip%=:"
      : "+v"(e0), "+v"(e1), "+v"(e2), "+v"(e3), "+v"(e4), "+v"(e5), "+v"(e6), "+v"(e7)
      : "v"(a), "s"(go)
      : "scc");
  acc[0][r] = e0; acc[1][r] = e1; acc[2][r] = e2; acc[3][r] = e3;
  acc[4][r] = e4; acc[5][r] = e5; acc[6][r] = e6; acc[7][r] = e7;
}
__device__ __forceinline__ float row16_max(float x) {
  x = fmaxf(x, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x128, 0xF, 0xF, false)));
  x = fmaxf(x, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x124, 0xF, 0xF, false)));
  x = fmaxf(x, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x122, 0xF, 0xF, false)));
  return fmaxf(x, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x121, 0xF, 0xF, false)));
}
__device__ __forceinline__ float row16_sum(float x) {
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x128, 0xF, 0xF, false));
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x124, 0xF, 0xF, false));
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x122, 0xF, 0xF, false));
  return x + __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x121, 0xF, 0xF, false));
}
// exponent e with 2^(e-1) <= |x| < 2^e (0 for x == 0)
__device__ __forceinline__ int exp_of(float amax) {
  return amax > 0.f ? (int)((__float_as_uint(amax) >> 23) & 0xFFu) - 126 : 0;
}

// Online-softmax state of the 4 rows (4 rg + r) a lane holds in the MFMA
// output layout, and the value accumulators acc[ct][r] (channel 16 ct + col).
struct ERowState {
  float m[4];   // reference (log2 domain); -inf until the row sees a live logit
  float l[4];   // this lane's partial sum of weights
  f32x4 acc[8];
};

// Lazy softmax update over x[c][r] (c = the two 16-token column halves of a
// 32-token step), then the weights of rows 4 rg + r, tokens 16 c + col, are
// written to this wave's LDS staging rows.  Returns nothing; updates st.
__device__ __forceinline__ void softmax_stage(ERowState& st, float (&x)[2][4], float* sp, int lane) {
  bool over = false;
#pragma unroll
  for (int c = 0; c < 2; ++c)
#pragma unroll
    for (int r = 0; r < 4; ++r) over |= x[c][r] > st.m[r] + kELazy;
  float alpha[4] = {1.f, 1.f, 1.f, 1.f};
  const bool grow = __builtin_amdgcn_ballot_w64(over) != 0;
  if (grow) {  // uniform: some row's max passed its reference
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float bm = row16_max(fmaxf(x[0][r], x[1][r]));
      const float mn = fmaxf(st.m[r], bm);
      alpha[r] = mn == -INFINITY ? 1.f : __builtin_amdgcn_exp2f(st.m[r] - mn);
      st.m[r] = mn;
      st.l[r] *= alpha[r];
    }
  }
  const uint32_t go = __builtin_amdgcn_readfirstlane(grow ? 1u : 0u);  // uniform: an SGPR operand
#pragma unroll
  for (int r = 0; r < 4; ++r) rescale_row<8>(st.acc, r, alpha[r], go);
  const int col = lane & 15, rg = lane >> 4;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const float ref = st.m[r] == -INFINITY ? 0.f : st.m[r] + kELazy;
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      const float p = __builtin_amdgcn_exp2f(x[c][r] - ref);  // 0 for -inf logits, <= 1 otherwise
      st.l[r] += p;
      sp[(4 * rg + r) * EPS + 16 * c + col] = p;
    }
  }
}

// Weights of this wave's 16 rows x 32 tokens from LDS into the MFMA A layout
// (lane: row lane % 16, tokens 8 (lane / 16) .. + 7) as fp16 hi and lo parts.
__device__ __forceinline__ void weights_a(const float* sp, int lane, f16x8& Ah, f16x8& Al) {
  const float* src = sp + (lane & 15) * EPS + 8 * (lane >> 4);
  const f32x4 a = *reinterpret_cast<const f32x4*>(src);
  const f32x4 b = *reinterpret_cast<const f32x4*>(src + 4);
  const float w[8] = {a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
  u32x4 hv, lv;
#pragma unroll
  for (int e2 = 0; e2 < 4; ++e2) {
    const uint2 hl = split2_f16(w[2 * e2], w[2 * e2 + 1]);
    hv[e2] = hl.x;
    lv[e2] = hl.y;
  }
  Ah = __builtin_bit_cast(f16x8, hv);
  Al = __builtin_bit_cast(f16x8, lv);
}

template <int KB, int VB, bool QJ>
__global__ __launch_bounds__(ENW * 64) void extend_kernel(EArgs a) {
  using R = ERec<KB, VB, QJ>;
  using LD = ELds<KB, VB, QJ>;
  extern __shared__ __attribute__((aligned(16))) unsigned char lds[];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int col = lane & 15, rg = lane >> 4;
  const int G = a.G;
  const int qtile = blockIdx.x % a.qtiles;
  const int bh = blockIdx.x / a.qtiles;
  const int b = bh / a.Hkv, h = bh % a.Hkv;
  const int cu0 = a.cu[b];
  int C = a.cu[b + 1] - cu0;
  C = C < 0 ? 0 : (C > a.max_chunk ? a.max_chunk : C);
  const int QT = EROWS / G;           // chunk tokens per tile
  const int tq0 = qtile * QT;
  if (tq0 >= C) return;                // uniform
  int P = a.prefix_lens[b];
  P = P < 0 ? 0 : (P > a.max_prefix ? a.max_prefix : P);

  uint2* s_pair = reinterpret_cast<uint2*>(lds + LD::pair);
  u32x4* s_sgn = reinterpret_cast<u32x4*>(lds + LD::sgn);
  float* s_uq = reinterpret_cast<float*>(lds + LD::rows);
  float* s_up = s_uq + EROWS;
  unsigned char* ring = lds + LD::ring;
  float* sp = reinterpret_cast<float*>(lds + LD::ps) + wave * 16 * EPS;
  uint16_t* s_ck = reinterpret_cast<uint16_t*>(lds + LD::ck);
  uint16_t* s_cv = reinterpret_cast<uint16_t*>(lds + LD::cv);
  float* st_q = reinterpret_cast<float*>(lds + LD::stage);
  float* st_p = st_q + EROWS * ED;

  // ---- tables: fp16 centroid pairs, fp16 +-1 patterns of sign bytes
  for (int i = tid; i < (1 << (2 * KB)); i += ENW * 64)
    s_pair[i] = make_uint2(a.dev.pair_lut_f16[2 * i], a.dev.pair_lut_f16[2 * i + 1]);
  if constexpr (QJ) {
    u32x4 w;
#pragma unroll
    for (int e = 0; e < 4; ++e)
      w[e] = (((tid >> (2 * e)) & 1) ? 0x3C00u : 0xBC00u) | ((((tid >> (2 * e + 1)) & 1) ? 0x3C00u : 0xBC00u) << 16);
    if (tid < 256) s_sgn[tid] = w;  // one entry per thread
  }

  // ---- rotate this wave's 16 query rows: q~ = D2 (H / sqrt d) D1 q into st_q
  // (lane holds coordinates 2 lane, 2 lane + 1; butterflies in-lane for index
  // bit 0, across lanes for bits 1..6)
  {
    const float s1 = lane_sign<1>(lane), s2 = lane_sign<2>(lane), s4 = lane_sign<4>(lane);
    const float s8 = lane_sign<8>(lane), s16 = lane_sign<16>(lane), s32 = lane_sign<32>(lane);
    const float d1a = a.dev.signs1[2 * lane], d1b = a.dev.signs1[2 * lane + 1];
    const float d2a = a.dev.signs2[2 * lane], d2b = a.dev.signs2[2 * lane + 1];
    const float inv = 1.0f / __builtin_sqrtf((float)ED);
    // the 16 rows' loads are issued together (one round trip), rows past the
    // chunk read as zeros
    uint32_t qraw[ERPW];
#pragma unroll
    for (int i = 0; i < ERPW; ++i) {
      const int r = wave * ERPW + i;
      const int tok = tq0 + r / G, hq = h * G + r % G;
      qraw[i] = tok < C ? *reinterpret_cast<const uint32_t*>(a.q + ((int64_t)(cu0 + tok) * a.Hq + hq) * ED + 2 * lane)
                        : 0u;  // uniform condition
    }
#pragma unroll
    for (int i = 0; i < ERPW; ++i) {
      const int r = wave * ERPW + i;
      const float x0 = __uint_as_float(qraw[i] << 16) * d1a;
      const float x1 = __uint_as_float(qraw[i] & 0xFFFF0000u) * d1b;
      float y0 = x0 + x1, y1 = x0 - x1;
      y0 = wht_xlane<1>(y0, s1);
      y1 = wht_xlane<1>(y1, s1);
      y0 = wht_xlane<2>(y0, s2);
      y1 = wht_xlane<2>(y1, s2);
      y0 = wht_xlane<4>(y0, s4);
      y1 = wht_xlane<4>(y1, s4);
      y0 = wht_xlane<8>(y0, s8);
      y1 = wht_xlane<8>(y1, s8);
      y0 = wht_xlane<16>(y0, s16);
      y1 = wht_xlane<16>(y1, s16);
      y0 = wht_xlane<32>(y0, s32);
      y1 = wht_xlane<32>(y1, s32);
      st_q[r * ED + 2 * lane] = y0 * inv * d2a;
      st_q[r * ED + 2 * lane + 1] = y1 * inv * d2b;
    }
  }
  __syncthreads();

  // ---- p = S q~ of the wave's rows on the matrix cores (A rows = rows,
  // fp16 hi/lo of q~ 2^-e per row; B = the context's tiles of 16 S)
  if constexpr (QJ) {
    const int arow = lane & 15, kq = lane >> 4;
    const int r = wave * ERPW + arow;
    float amax = 0.f;
#pragma unroll
    for (int j = 0; j < ED / 4; ++j) amax = fmaxf(amax, fabsf(st_q[r * ED + 32 * (j / 8) + 8 * kq + (j % 8)]));
    amax = fmaxf(amax, __shfl_xor(amax, 16, 64));
    amax = fmaxf(amax, __shfl_xor(amax, 32, 64));
    const int e = exp_of(amax);
    const float sc = __builtin_ldexpf(1.0f, -e);
    f16x8 ah[EKT], al[EKT];
#pragma unroll
    for (int kt = 0; kt < EKT; ++kt)
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        _Float16 hh, ll;
        split_f16(st_q[r * ED + 32 * kt + 8 * kq + i] * sc, hh, ll);
        ah[kt][i] = hh;
        al[kt][i] = ll;
      }
    // the output row 4 rg + rr belongs to row wave * 16 + 4 rg + rr; its
    // scale exponent comes from the lane holding that row in the A layout
    int eo[4];
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) eo[rr] = __shfl(e, 4 * rg + rr, 64);
    const float unscale = 1.0f / (float)(1 << kSScaleLog2);
    for (int nt = 0; nt < ED / 16; ++nt) {
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kt = 0; kt < EKT; ++kt) {
        const size_t tb = (((size_t)nt * EKT + kt) * 2) * 64 * 8;
        const f16x8 bhi = *reinterpret_cast<const f16x8*>(a.dev.s_tiles + tb + lane * 8);
        const f16x8 blo = *reinterpret_cast<const f16x8*>(a.dev.s_tiles + tb + 512 + lane * 8);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(ah[kt], bhi, acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(ah[kt], blo, acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(al[kt], bhi, acc, 0, 0, 0);
      }
#pragma unroll
      for (int rr = 0; rr < 4; ++rr)
        st_p[(wave * ERPW + 4 * rg + rr) * ED + 16 * nt + col] = __builtin_ldexpf(acc[rr] * unscale, eo[rr]);
    }
  }
  __syncthreads();

  // ---- score A operands: q~ log2(e) sm_scale and p kappa log2(e) sm_scale,
  // each scaled per row by a power of two into [2^13, 2^14) and split into
  // fp16 hi / lo; the raw bf16 query for the chunk's exact scores
  f16x8 aqh[EKT], aql[EKT], aph[EKT], apl[EKT];
  bf16x8 ac[EKT];
  {
    const int arow = lane & 15, kq = lane >> 4;
    const int r = wave * ERPW + arow;
    const float ls = a.logit_scale;
    const float lk = 1.2533141373155003f / (float)ED * a.logit_scale;  // sqrt(pi/2) / d
    float mq = 0.f, mp = 0.f;
#pragma unroll
    for (int j = 0; j < ED / 4; ++j) {
      const int c = 32 * (j / 8) + 8 * kq + (j % 8);
      mq = fmaxf(mq, fabsf(st_q[r * ED + c]));
      if constexpr (QJ) mp = fmaxf(mp, fabsf(st_p[r * ED + c]));
    }
    mq = fmaxf(mq, __shfl_xor(mq, 16, 64));
    mq = fmaxf(mq, __shfl_xor(mq, 32, 64));
    mp = fmaxf(mp, __shfl_xor(mp, 16, 64));
    mp = fmaxf(mp, __shfl_xor(mp, 32, 64));
    const int eq = exp_of(mq * ls), ep = exp_of(mp * lk);
    const float sq = __builtin_ldexpf(ls, 14 - eq), spp = __builtin_ldexpf(lk, 14 - ep);
#pragma unroll
    for (int kt = 0; kt < EKT; ++kt)
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        _Float16 hh, ll;
        split_f16(st_q[r * ED + 32 * kt + 8 * kq + i] * sq, hh, ll);
        aqh[kt][i] = hh;
        aql[kt][i] = ll;
        if constexpr (QJ) {
          split_f16(st_p[r * ED + 32 * kt + 8 * kq + i] * spp, hh, ll);
          aph[kt][i] = hh;
          apl[kt][i] = ll;
        } else {
          aph[kt][i] = (_Float16)0.f;
          apl[kt][i] = (_Float16)0.f;
        }
      }
    if (kq == 0) {
      s_uq[r] = __builtin_ldexpf(1.0f, eq - 14);
      s_up[r] = __builtin_ldexpf(1.0f, ep - 14);
    }
    const int tok = tq0 + r / G, hq = h * G + r % G;
#pragma unroll
    for (int kt = 0; kt < EKT; ++kt) {
      u32x4 w = {0u, 0u, 0u, 0u};
      if (tok < C) w = *reinterpret_cast<const u32x4*>(a.q + ((int64_t)(cu0 + tok) * a.Hq + hq) * ED + 32 * kt + 8 * kq);
      ac[kt] = __builtin_bit_cast(bf16x8, w);
    }
  }
  __syncthreads();  // the staging area becomes the B tiles; s_uq / s_up are complete

  // the four rows 4 rg + r this lane holds in the MFMA output layout
  float uq[4], up[4];
  int rtok[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int row = wave * ERPW + 4 * rg + r;
    uq[r] = s_uq[row];
    up[r] = s_up[row];
    rtok[r] = tq0 + row / G;
  }
  ERowState st;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    st.m[r] = -INFINITY;
    st.l[r] = 0.f;
  }
#pragma unroll
  for (int ct = 0; ct < 8; ++ct) st.acc[ct] = f32x4{0.f, 0.f, 0.f, 0.f};

  // ---------------------------------------------------------- the prefix
  // A software pipeline over 32-token steps with one barrier per step: the
  // iteration of step s stores the records of step s + 2 into its ring slot
  // (three slots), issues the loads of step s + 3, computes the scores of
  // step s, builds the B tiles of step s + 1 into the tile buffer step s does
  // not use (between the score and value products, in the same basic block,
  // so the compiler can interleave the build's VALU and LDS work with the
  // matrix products), and finishes step s.  The barrier that ends the
  // iteration orders its writes before the next iteration's reads: a ring
  // slot is rewritten two iterations after its step was built and one after
  // it was computed, a tile buffer one iteration after its step was computed.
  // Measured on the prefill workload: 2017 us with four-wave workgroups and
  // two barriers per step, 1625 us with eight waves, 1481 us pipelined,
  // 1433 us with the build placed between the products, 1402 us with the
  // two-value fp16 splits, 1370 us with the copy-free rescale.
  const int nsteps = (P + 31) / 32;
  const int32_t* btrow = a.bt + (int64_t)b * a.max_blocks;
  // 16-byte pieces of a step's two records: thread t copies pieces t, t + ENW * 64, ..
  constexpr int NPC = 2 * R::pieces;
  constexpr int NFJ = (NPC + ENW * 64 - 1) / (ENW * 64);
  auto fetch = [&](int st, u32x4 (&pf)[NFJ]) {
#pragma unroll
    for (int j = 0; j < NFJ; ++j) {
      const int pc = tid + j * ENW * 64;
      pf[j] = u32x4{0u, 0u, 0u, 0u};
      if (pc < NPC) {
        const int rr = pc / R::pieces, off = (pc % R::pieces) * 16;
        const int bi = 2 * st + rr;
        const int blk = (bi < a.max_blocks && 16 * bi < P) ? btrow[bi] : -1;
        if (blk >= 0 && (int64_t)blk < a.pool_blocks)
          pf[j] = __builtin_nontemporal_load(
              reinterpret_cast<const u32x4*>(a.pool + ((int64_t)blk * a.Hkv + h) * a.rec + off));
      }
    }
  };
  auto ring_at = [&](int st) -> unsigned char* { return ring + (st % 3) * LD::ring_slot; };
  auto store_ring = [&](int st, const u32x4 (&pf)[NFJ]) {
    unsigned char* rg = ring_at(st);
#pragma unroll
    for (int j = 0; j < NFJ; ++j) {
      const int pc = tid + j * ENW * 64;
      if (pc < NPC) *reinterpret_cast<u32x4*>(rg + pc * 16) = pf[j];
    }
  };
  // the shared B tiles of step st from its ring slot (512 slots of each kind)
  auto build = [&](int st) {
    const unsigned char* rg = ring_at(st);
    u32x4* kcb = reinterpret_cast<u32x4*>(lds + LD::kc + (st & 1) * LD::kc_buf);
    u32x4* ksb = reinterpret_cast<u32x4*>(lds + LD::ks + (st & 1) * LD::ks_buf);
    u32x4* vtb = reinterpret_cast<u32x4*>(lds + LD::vt + (st & 1) * LD::vt_buf);
    // one slot of each kind per thread
    const int t_base = 32 * st;
#pragma unroll
    for (int j = 0; j < 512 / (ENW * 64); ++j) {
      const int slot = tid + j * ENW * 64;  // (half, kt, lane) = (slot / 256, (slot / 64) % 4, slot % 64)
      const int half = slot >> 8, kt = (slot >> 6) & 3, ln = slot & 63;
      const int n = ln & 15, kq = ln >> 4;
      const unsigned char* rec = rg + half * R::bytes;
      // 8 codes (coordinates 32 kt + 8 kq ..) of token n
      const int bit0 = KB * (32 * kt + 8 * kq);
      const unsigned char* cs = rec + R::kcodes + n * (KB * ED / 8);
      const uint32_t* cw = reinterpret_cast<const uint32_t*>(cs + (bit0 >> 5) * 4);
      uint32_t wv = cw[0];
      if constexpr (KB == 3) {
        const int sh = bit0 & 31;
        if (sh + 24 > 32) wv = __builtin_amdgcn_alignbit(cw[1], cw[0], sh);
        else wv >>= sh;
      } else {
        wv >>= (bit0 & 31);
      }
      u32x4 bh, bl;
#pragma unroll
      for (int pi = 0; pi < 4; ++pi) {
        const uint2 pe = s_pair[(wv >> (2 * KB * pi)) & ((1u << (2 * KB)) - 1u)];
        bh[pi] = pe.x;
        bl[pi] = pe.y;
      }
      u32x4* kcw = kcb + ((half * EKT + kt) * 2) * 64 + ln;
      kcw[0] = bh;
      kcw[64] = bl;
      if constexpr (QJ) {
        const uint32_t byte = rec[R::kqjl + n * (ED / 8) + 4 * kt + kq];
        ksb[(half * EKT + kt) * 64 + ln] = s_sgn[byte];
      }
      // values: channel tile ct = slot / 64, channel 16 ct + n, tokens 8 kq .. + 7
      // (record kq / 2, slots 8 (kq % 2) .. + 7)
      {
        const int ct = slot >> 6;
        const int c = 16 * ct + n;
        const unsigned char* vr = rg + (kq >> 1) * R::bytes;
        const int s0 = 8 * (kq & 1);
        constexpr int CPB = 8 / VB;              // codes per byte
        const int f = c / CPB;                   // byte of the code stream
        const int sh = 8 * (f & 3) + VB * (c % CPB);
        const u32x4* cp = reinterpret_cast<const u32x4*>(vr + R::vcodes + ((f >> 2) * 16 + s0) * 4);
        const u32x4* mp = reinterpret_cast<const u32x4*>(vr + R::vmeta + ((c >> 5) * 16 + s0) * 4);
        const u32x4 c0 = cp[0], c1 = cp[1], m0 = mp[0], m1 = mp[1];
        const uint32_t cd[8] = {c0[0], c0[1], c0[2], c0[3], c1[0], c1[1], c1[2], c1[3]};
        const uint32_t md[8] = {m0[0], m0[1], m0[2], m0[3], m1[0], m1[1], m1[2], m1[3]};
        u32x4 vh, vl;
#pragma unroll
        for (int e2 = 0; e2 < 4; ++e2) {
          float vv[2];
#pragma unroll
          for (int u = 0; u < 2; ++u) {
            const int e = 2 * e2 + u;
            const int tok = t_base + 16 * (kq >> 1) + s0 + e;
            const float qv = (float)((cd[e] >> sh) & ((1u << VB) - 1u));
            const f16x2 sz = __builtin_bit_cast(f16x2, md[e]);  // {s, z}
            const float v = __builtin_fmaf(qv, (float)sz[0], (float)sz[1]);
            vv[u] = (tok < P) ? v : 0.f;  // tokens past the prefix (or in a skipped block) hold no data
          }
          const uint2 hl = split2_f16(vv[0], vv[1]);
          vh[e2] = hl.x;
          vl[e2] = hl.y;
        }
        u32x4* vtw = vtb + (ct * 2) * 64 + ln;
        vtw[0] = vh;
        vtw[64] = vl;
      }
    }
  };
  u32x4 pf[NFJ];
  if (nsteps > 0) {
    fetch(0, pf);
    store_ring(0, pf);
  }
  if (nsteps > 1) {
    fetch(1, pf);
    store_ring(1, pf);
  }
  if (nsteps > 2) fetch(2, pf);
  __syncthreads();
  if (nsteps > 0) build(0);
  __syncthreads();
  for (int s = 0; s < nsteps; ++s) {
    // unconditional: past the prefix the loads read nothing (zeros), and the
    // ring slot and tile buffer written are never read
    store_ring(s + 2, pf);
    fetch(s + 3, pf);
    const u32x4* s_kc = reinterpret_cast<const u32x4*>(lds + LD::kc + (s & 1) * LD::kc_buf);
    const u32x4* s_ks = reinterpret_cast<const u32x4*>(lds + LD::ks + (s & 1) * LD::ks_buf);
    const u32x4* s_vt = reinterpret_cast<const u32x4*>(lds + LD::vt + (s & 1) * LD::vt_buf);
    const int t_base = 32 * s;
    // ---- scores of the wave's 16 rows against the step's 32 tokens
    float x[2][4];
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      f32x4 am = {0.f, 0.f, 0.f, 0.f}, aq = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kt = 0; kt < EKT; ++kt) {
        const f16x8 bh = __builtin_bit_cast(f16x8, s_kc[((half * EKT + kt) * 2) * 64 + lane]);
        const f16x8 bl = __builtin_bit_cast(f16x8, s_kc[((half * EKT + kt) * 2 + 1) * 64 + lane]);
        am = __builtin_amdgcn_mfma_f32_16x16x32_f16(aqh[kt], bh, am, 0, 0, 0);
        am = __builtin_amdgcn_mfma_f32_16x16x32_f16(aqh[kt], bl, am, 0, 0, 0);
        am = __builtin_amdgcn_mfma_f32_16x16x32_f16(aql[kt], bh, am, 0, 0, 0);
        if constexpr (QJ) {
          const f16x8 bs = __builtin_bit_cast(f16x8, s_ks[(half * EKT + kt) * 64 + lane]);
          aq = __builtin_amdgcn_mfma_f32_16x16x32_f16(aph[kt], bs, aq, 0, 0, 0);
          aq = __builtin_amdgcn_mfma_f32_16x16x32_f16(apl[kt], bs, aq, 0, 0, 0);
        }
      }
      const unsigned char* rec = ring_at(s) + half * R::bytes;
      const int tok = t_base + 16 * half + col;
      const int bi = 2 * s + half;
      const int blk = 16 * bi < P ? btrow[bi] : -1;  // uniform
      const bool live = tok < P && blk >= 0 && (int64_t)blk < a.pool_blocks;
      const uint32_t km = QJ ? *reinterpret_cast<const uint32_t*>(rec + R::kmeta + col * 4)
                             : (uint32_t)*reinterpret_cast<const uint16_t*>(rec + R::kmeta + col * 2);
      const float nv = f16_bits_to_f32((uint16_t)(km & 0xFFFFu));
      const float gv = QJ ? f16_bits_to_f32((uint16_t)(km >> 16)) : 0.f;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        float v = am[r] * uq[r];
        if constexpr (QJ) v = __builtin_fmaf(gv * up[r], aq[r], v);
        x[half][r] = live ? nv * v : -INFINITY;
      }
    }
    build(s + 1);
    softmax_stage(st, x, sp, lane);
    __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): the weights are in LDS
    __builtin_amdgcn_wave_barrier();
    f16x8 Ah, Al;
    weights_a(sp, lane, Ah, Al);
#pragma unroll
    for (int ct = 0; ct < 8; ++ct) {
      const f16x8 bh = __builtin_bit_cast(f16x8, s_vt[(ct * 2) * 64 + lane]);
      const f16x8 bl = __builtin_bit_cast(f16x8, s_vt[(ct * 2 + 1) * 64 + lane]);
      st.acc[ct] = __builtin_amdgcn_mfma_f32_16x16x32_f16(Ah, bh, st.acc[ct], 0, 0, 0);
      st.acc[ct] = __builtin_amdgcn_mfma_f32_16x16x32_f16(Ah, bl, st.acc[ct], 0, 0, 0);
      st.acc[ct] = __builtin_amdgcn_mfma_f32_16x16x32_f16(Al, bh, st.acc[ct], 0, 0, 0);
    }
    __syncthreads();
  }

  // ------------------------------------------------------- the chunk itself
  const int kend = min(C, tq0 + QT);  // keys this tile's queries can see
  for (int j0 = 0; j0 < kend; j0 += 32) {
    __syncthreads();  // every wave is done with the previous tiles
    // K tile [32][D] bf16 and V tile transposed [D][32] fp16
#pragma unroll
    for (int j = 0; j < 512 / (ENW * 64); ++j) {
      const int pc = tid + j * ENW * 64;  // 512 pieces of 16 bytes: token pc / 16, channels 8 (pc % 16) ..
      const int t = pc >> 4, c8 = (pc & 15) * 8;
      const int tok = j0 + t;
      u32x4 kw = {0u, 0u, 0u, 0u}, vw = {0u, 0u, 0u, 0u};
      if (tok < C) {
        const int64_t off = ((int64_t)(cu0 + tok) * a.Hkv + h) * ED + c8;
        kw = *reinterpret_cast<const u32x4*>(a.k + off);
        vw = *reinterpret_cast<const u32x4*>(a.v + off);
      }
      *reinterpret_cast<u32x4*>(s_ck + t * EKR + c8) = kw;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float lo = __uint_as_float(vw[e] << 16), hi = __uint_as_float(vw[e] & 0xFFFF0000u);
        s_cv[(c8 + 2 * e) * EVS + t] = f32_to_f16_bits(lo);
        s_cv[(c8 + 2 * e + 1) * EVS + t] = f32_to_f16_bits(hi);
      }
    }
    __syncthreads();
    float x[2][4];
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
      const int kq = lane >> 4;
#pragma unroll
      for (int kt = 0; kt < EKT; ++kt) {
        const bf16x8 bk = *reinterpret_cast<const bf16x8*>(s_ck + (16 * half + col) * EKR + 32 * kt + 8 * kq);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ac[kt], bk, acc, 0, 0, 0);
      }
      const int key = j0 + 16 * half + col;
#pragma unroll
      for (int r = 0; r < 4; ++r) x[half][r] = (key < C && key <= rtok[r]) ? acc[r] * a.logit_scale : -INFINITY;
    }
    softmax_stage(st, x, sp, lane);
    __builtin_amdgcn_s_waitcnt(0xc07f);
    __builtin_amdgcn_wave_barrier();
    f16x8 Ah, Al;
    weights_a(sp, lane, Ah, Al);
    const int kq = lane >> 4;
#pragma unroll
    for (int ct = 0; ct < 8; ++ct) {
      const f16x8 bv = *reinterpret_cast<const f16x8*>(s_cv + (16 * ct + col) * EVS + 8 * kq);
      st.acc[ct] = __builtin_amdgcn_mfma_f32_16x16x32_f16(Ah, bv, st.acc[ct], 0, 0, 0);
      st.acc[ct] = __builtin_amdgcn_mfma_f32_16x16x32_f16(Al, bv, st.acc[ct], 0, 0, 0);
    }
  }

  // ---------------------------------------------------------------- output
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const float l = row16_sum(st.l[r]);
    const int row = wave * ERPW + 4 * rg + r;
    const int tok = tq0 + row / G, hq = h * G + row % G;
    if (tok < C) {
      float* o = a.out + ((int64_t)(cu0 + tok) * a.Hq + hq) * ED;
#pragma unroll
      for (int ct = 0; ct < 8; ++ct) o[16 * ct + col] = l > 0.f ? st.acc[ct][r] / l : 0.f;
    }
  }
}

template <int KB, int VB, bool QJ>
hipError_t launch_e(const EArgs& a, int grid, hipStream_t stream) {
  auto kern = extend_kernel<KB, VB, QJ>;
  using LD = ELds<KB, VB, QJ>;
  static std::mutex mu;
  static bool granted[16] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= 16) return hipErrorInvalidDevice;
  {
    std::lock_guard<std::mutex> lock(mu);
    if (!granted[dev]) {
      e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern), hipFuncAttributeMaxDynamicSharedMemorySize,
                              LD::total);
      if (e != hipSuccess) return e;
      granted[dev] = true;
    }
  }
  hipLaunchKernelGGL(kern, dim3(grid), dim3(ENW * 64), LD::total, stream, a);
  return hipGetLastError();
}

template <int KB, int VB, bool QJ>
bool layout_matches(const Layout& l) {
  using R = ERec<KB, VB, QJ>;
  return l.kcodes == R::kcodes && l.kqjl == R::kqjl && l.kmeta == R::kmeta && l.vcodes == R::vcodes &&
         l.vmeta == R::vmeta && l.bytes == R::bytes;
}

template <bool QJ>
hipError_t dispatch_e(const EArgs& a, int kb, int vb, const Layout& lay, int grid, hipStream_t s) {
#define TQ_EXT_CASE(KB_, VB_)                                                        \
  if (kb == KB_ && vb == VB_) {                                                      \
    if (!layout_matches<KB_, VB_, QJ>(lay)) return hipErrorInvalidValue;            \
    return launch_e<KB_, VB_, QJ>(a, grid, s);                                       \
  }
  TQ_EXT_CASE(2, 2)
  TQ_EXT_CASE(2, 4)
  TQ_EXT_CASE(3, 2)
  TQ_EXT_CASE(3, 4)
  TQ_EXT_CASE(4, 2)
  TQ_EXT_CASE(4, 4)
#undef TQ_EXT_CASE
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_extend(const tq_extend_args* x, hipStream_t stream) {
  const tq_ctx* c = x->ctx;
  EArgs a{};
  a.q = reinterpret_cast<const uint16_t*>(x->q);
  a.k = reinterpret_cast<const uint16_t*>(x->k);
  a.v = reinterpret_cast<const uint16_t*>(x->v);
  a.cu = x->cu_chunk;
  a.B = x->batch;
  a.Hq = x->num_q_heads;
  a.Hkv = x->num_kv_heads;
  a.G = a.Hq / a.Hkv;
  a.max_chunk = x->max_chunk;
  a.pool = reinterpret_cast<const uint8_t*>(x->pool);
  a.pool_blocks = x->pool_blocks;
  a.rec = c->lay.bytes;
  a.dev = c->dev;
  a.bt = x->block_tables;
  a.max_blocks = x->max_blocks_per_seq;
  a.prefix_lens = x->prefix_lens;
  a.max_prefix = x->max_prefix_len;
  const float sm = x->sm_scale > 0.f ? x->sm_scale : 1.0f / std::sqrt((float)ED);
  a.logit_scale = sm * 1.4426950408889634f;
  a.out = x->out;
  a.qtiles = (x->max_chunk + EROWS / a.G - 1) / (EROWS / a.G);
  const int64_t grid = (int64_t)a.B * a.Hkv * a.qtiles;
  if (grid == 0) return hipSuccess;
  if (grid > 0x7FFFFFFF) return hipErrorInvalidValue;
  return c->qjl ? dispatch_e<true>(a, c->kb, c->vb, c->lay, (int)grid, stream)
                : dispatch_e<false>(a, c->kb, c->vb, c->lay, (int)grid, stream);
}

}  // namespace tq
