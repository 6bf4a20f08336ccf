// Decode attention over the compressed paged cache for gfx950.
//
// Roadmap §3.2 (the vLLM v2 decode design): grouped query heads share one pass
// over a KV head, the query is rotated once and scores come straight from the
// codes through per-query tables, and the softmax runs in the exp2 domain;
// Roadmap §3.1 / §7: the grid is fixed for graph capture and the split
// partials live in a caller-provided workspace; Roadmap §4.4: empty rows and
// empty splits must not produce NaN or divide by zero.
//
// One or two launches on one stream:
//   split   : a persistent grid walks the work items (sequence, KV head,
//             split); each workgroup rotates and projects the item's queries
//             (q~ = D2 (H/sqrt d) D1 q, p = S q~), streams one chunk of cached
//             tokens (or the recent full-precision window) and leaves
//             (m, l, acc[d]) per query head, or the normalised output itself
//             when every sequence is a single split;
//   combine : log-sum-exp merge of the splits (empty splits contribute 0),
//             only when some sequence has more than one split.
//
// In `split`, a wave consumes 32 tokens (two paged blocks) per step:
//   scores   [G x 16] per block = q~ . c[idx] + p . (2 sigma - 1) on
//            v_mfma_f32_16x16x32_bf16: A = q~ (bf16 hi rows and lo rows stacked
//            in the 16 MFMA rows), B = centroid hi / lo of the packed codes
//            fetched two codes at a time from an LDS pair table, and B = +-1
//            from an LDS byte table for the sign bits (MSE-only keys: the
//            first product alone);
//   softmax  running max / sum per head in the exp2 domain;
//   values   acc[(group, head)][channel] += (p s)_hi,lo . (sigma q 2^-24) on
//            v_mfma_f32_16x16x32_f16, each code placed at mantissa bit 4 (or
//            bit 6 for half of the 2-bit codes) of an fp16 subnormal, with the
//            zero-points folded into one
//            per-(group, head) scalar; only the rows of each column's own
//            group are kept at the end.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <mutex>

#include <type_traits>

#include "tq_common.hip.h"
#include "tq_internal.h"

#ifndef TQ_DECODE_QJL
#error "compile with -DTQ_DECODE_QJL=1 (keys with the QJL sketch) or 0 (MSE-only keys)"
#endif

namespace tq {

constexpr int kMaxG = 8;

struct DArgs {
  const void* q;
  int q_bf16;
  int B, Hq, Hkv, G;
  const uint8_t* pool[2];
  int64_t pool_blocks[2];
  int64_t rec[2];
  Layout lay[2];
  DevTables dev[2];
  const int8_t* seq_preset;
  const int32_t* bt;
  int max_blocks;
  const int32_t* seq_lens;
  int max_seq_len;
  const uint16_t* rk;
  const uint16_t* rv;
  const int32_t* rlens;
  int W;
  float logit_scale;  // sm_scale * log2(e)
  float inv_logit_scale;
  float sm_scale;
  int chunk;
  int splits_cap;
  float* part;   // [B][Hq][splits_cap][D + 2]
  float* out;
  float* scores;
  int scores_stride;
  int direct;  // every sequence has at most one split: write the normalised output, no partials
};

__device__ __forceinline__ int seq_cached(const DArgs& a, int b) {
  int L = a.seq_lens[b];
  L = L < 0 ? 0 : L;
  L = L > a.max_seq_len ? a.max_seq_len : L;
  return L;
}
__device__ __forceinline__ int seq_recent(const DArgs& a, int b) {
  if (!a.rk) return 0;
  int R = a.rlens[b];
  return R < 0 ? 0 : (R > a.W ? a.W : R);
}
__device__ __forceinline__ int seq_splits(const DArgs& a, int b) {
  return (seq_cached(a, b) + a.chunk - 1) / a.chunk + (seq_recent(a, b) > 0 ? 1 : 0);
}
__device__ __forceinline__ int seq_preset_of(const DArgs& a, int b) {
  return a.seq_preset ? (a.seq_preset[b] != 0 ? 1 : 0) : 0;
}

// ---------------------------------------------------------------------------
// split
// ---------------------------------------------------------------------------
constexpr int kMaxChunk = 8192;  // largest chunk_tokens (block ids of a chunk are staged in LDS)
// Online softmax with a lazily moved reference: a head's reference m (kept
// in m_run) only moves when a block's max exceeds m + kLazyMax, and weights
// are exp2(x - m - kLazyMax) <= 1.  Every weight, l and acc of the stream
// carries the same 2^-kLazyMax factor, which cancels in acc / l and in the
// merge of partials (a partial reports m + kLazyMax as its reference, like
// the exact-max partials of the recent window); the rescale of the
// accumulators becomes rare.
constexpr float kLazyMax = 2.0f;

// Compile-time geometry of one (block, KV head) record (the same byte layout
// the host computes) and of one 32-token step = two records.  QJ = false:
// MSE-only keys (no sign bits, key metadata = fp16 n per slot).
template <int D, int KB, int VB, bool QJ>
struct Rec {
  static constexpr int kcodes = 0;
  static constexpr int kqjl = kcodes + 16 * (KB * D / 8);
  static constexpr int kmeta = kqjl + (QJ ? 16 * (D / 8) : 0);
  static constexpr int kmeta_slot = QJ ? 4 : 2;  // bytes of one slot's key metadata
  static constexpr int vcodes = kmeta + 16 * kmeta_slot;
  static constexpr int vmeta = vcodes + (VB * D / 8) * 16;
  static constexpr int bytes = vmeta + (D / 32) * 64;
  static constexpr int slot = 2 * bytes;              // LDS bytes of one ring slot (one step)
  // records small enough for eight query heads per KV head to run 8-wave
  // workgroups (see split_waves)
  static constexpr bool kWide = D == 128 && bytes <= 2400;
};

// Waves per split workgroup.  d = 128 with up to 4 query heads per KV head
// fits two waves per SIMD (<= 256 VGPRs), so one 8-wave workgroup fills a CU
// and its waves share one item.  With eight query heads the value
// accumulators double; for records of at most 2400 bytes (2- and 3-bit keys,
// 4-bit keys with 2-bit values or without the sketch) the score A operands
// then move to LDS (lds_a) and the ring to two steps, which brings the
// kernel under 256 VGPRs and to 8-wave workgroups as well (the decode
// workload's shape at 64 query heads: 128 -> 102 us).  MSE-only keys of up to
// 4 bits with the Lloyd-Max codebook and four query heads per KV head carry
// no sketch registers: with the A operands in LDS and a two-step ring they fit
// three waves per SIMD (<= 168 VGPRs), so 12-wave workgroups share an item
// (the MSE-only decode workload: 65 -> 62 us); the equally spaced codebook's
// variant would spill there and keeps 8.  The other variants run one wave per
// SIMD.
template <int D, int GP, int KB, int VB, bool QJ, bool UN>
constexpr int split_waves() {
  return (D == 128 && GP == 4) ? (!QJ && !UN && KB <= 4 && Rec<D, KB, VB, QJ>::kWide ? 12 : 8)
                               : (D == 128 && GP == 8 && Rec<D, KB, VB, QJ>::kWide) ? 8 : 4;
}
// ring depth (steps in flight + 1) of each wave
template <int D, int GP, int KB, int VB, bool QJ, bool UN>
constexpr int ring_depth() {
  return split_waves<D, GP, KB, VB, QJ, UN>() == 12 || (D == 128 && GP == 8 && Rec<D, KB, VB, QJ>::kWide)
             ? 2
             : (D == 128 && KB <= 4 ? 3 : 2);
}
// the item's score A operands live in LDS (one copy the waves share) instead
// of registers
template <int D, int GP, int KB, int VB, bool QJ, bool UN>
constexpr bool lds_a() {
  return split_waves<D, GP, KB, VB, QJ, UN>() == 12 || (GP == 8 && split_waves<D, GP, KB, VB, QJ, UN>() == 8);
}

template <int D, int GP, int KB, int VB, bool QJ, bool UN>
struct SplitLds {
  static_assert(Rec<D, KB, VB, QJ>::bytes % 16 == 0, "record size");
  // per-wave softmax weights [GP][32]; with GP = 4 the idle lanes 32-63 store
  // theirs to a second, never-read copy so that the store needs no lane mask
  static constexpr int kPWave = GP * 32 * (GP == 4 ? 2 : 1);
  static constexpr int NW = split_waves<D, GP, KB, VB, QJ, UN>();
  static constexpr int kPBytes = NW * kPWave * 4;
  static constexpr int kStatBytes = NW * GP * 2 * 4;
  static constexpr int kBlkBytes = (kMaxChunk / 16 + 16) * 4;
  static constexpr int kRingBytes = NW * ring_depth<D, GP, KB, VB, QJ, UN>() * Rec<D, KB, VB, QJ>::slot;
  static constexpr int kMergeBytes = NW * GP * D * 4;  // overlays the ring after the stream
  static constexpr int kMainBytes = kRingBytes > kMergeBytes ? kRingBytes : kMergeBytes;
  static constexpr int kABytes = lds_a<D, GP, KB, VB, QJ, UN>() ? (D / 32) * 3 * 64 * 16 : 0;  // score A operands
  static constexpr int kMainOffset = kPBytes + kStatBytes + kBlkBytes + kABytes;
  static_assert(kMainOffset % 16 == 0, "ring alignment");
  static constexpr int total = kMainOffset + kMainBytes;
  // with the static tables (< 16 KB) the workgroup must fit a CU's 160 KB
  static_assert(total <= (160 - 16) * 1024, "split workgroup LDS");
};

// Row-wide (16-lane) reductions with DPP row rotations.
template <int kCtrl>
__device__ __forceinline__ float dpp_ror(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), kCtrl, 0xF, 0xF, false));
}
__device__ __forceinline__ float row_sum16(float x) {
  x += dpp_ror<0x128>(x);  // row_ror:8
  x += dpp_ror<0x124>(x);  // row_ror:4
  x += dpp_ror<0x122>(x);  // row_ror:2
  x += dpp_ror<0x121>(x);  // row_ror:1
  return x;
}
// Max over each 16-lane row of four values at once; the four chains are
// interleaved so every DPP read is 3 instructions after its producer.
__device__ __forceinline__ void row_max16x4(float& a, float& b, float& c, float& d) {
  asm volatile(
      "s_nop 1\n\t"
      "v_max_f32_dpp %0, %0, %0 row_ror:8 row_mask:0xf bank_mask:0xf\n\t"
      "v_max_f32_dpp %1, %1, %1 row_ror:8 row_mask:0xf bank_mask:0xf\n\t"
      "v_max_f32_dpp %2, %2, %2 row_ror:8 row_mask:0xf bank_mask:0xf\n\t"
      "v_max_f32_dpp %3, %3, %3 row_ror:8 row_mask:0xf bank_mask:0xf\n\t"
      "v_max_f32_dpp %0, %0, %0 row_ror:4 row_mask:0xf bank_mask:0xf\n\t"
      "v_max_f32_dpp %1, %1, %1 row_ror:4 row_mask:0xf bank_mask:0xf\n\t"
      "v_max_f32_dpp %2, %2, %2 row_ror:4 row_mask:0xf bank_mask:0xf\n\t"
      "v_max_f32_dpp %3, %3, %3 row_ror:4 row_mask:0xf bank_mask:0xf\n\t"
      "v_max_f32_dpp %0, %0, %0 row_ror:2 row_mask:0xf bank_mask:0xf\n\t"
      "v_max_f32_dpp %1, %1, %1 row_ror:2 row_mask:0xf bank_mask:0xf\n\t"
      "v_max_f32_dpp %2, %2, %2 row_ror:2 row_mask:0xf bank_mask:0xf\n\t"
      "v_max_f32_dpp %3, %3, %3 row_ror:2 row_mask:0xf bank_mask:0xf\n\t"
      "v_max_f32_dpp %0, %0, %0 row_ror:1 row_mask:0xf bank_mask:0xf\n\t"
      "v_max_f32_dpp %1, %1, %1 row_ror:1 row_mask:0xf bank_mask:0xf\n\t"
      "v_max_f32_dpp %2, %2, %2 row_ror:1 row_mask:0xf bank_mask:0xf\n\t"
      "v_max_f32_dpp %3, %3, %3 row_ror:1 row_mask:0xf bank_mask:0xf\n\t"
      "s_nop 1"
      : "+v"(a), "+v"(b), "+v"(c), "+v"(d));
}
__device__ __forceinline__ float lane_swap32_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float lane_swap16_sum(float x) {
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ uint32_t lds_offset(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}
// Wave-uniform copy of a 32-bit value, zero-extended when widened (the
// builtin returns a signed int, which would sign-extend the low half of an
// address).
__device__ __forceinline__ uint32_t uniform_u32(uint32_t x) {
  return (uint32_t)__builtin_amdgcn_readfirstlane((int)x);
}
// Direct global -> LDS copy of 16 bytes per lane: lane l's bytes land at LDS
// byte address m0 + 16 l.  Issued as inline assembly so that the compiler does
// not fence every later LDS read on it; completion is awaited explicitly with
// wait_vmcnt below.
__device__ __forceinline__ void dma16(uint32_t lds_byte_addr, uint64_t sbase, uint32_t voff) {
  asm volatile(
      "s_mov_b32 m0, %0\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %2, %1"
      :
      : "s"(uniform_u32(lds_byte_addr)),
        "s"(((uint64_t)uniform_u32((uint32_t)(sbase >> 32)) << 32) | (uint64_t)uniform_u32((uint32_t)sbase)),
        "v"(voff)
      : "memory");
}
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0)" : : "n"(N) : "memory");
}
// (y & mask) | c.  `c` is kept opaque to the compiler (see opaque_u32) so
// that it selects one v_and_or_b32 instead of two literal-operand VOP2 ops;
// the instruction stays compiler-generated so MFMA operand hazards are seen.
__device__ __forceinline__ uint32_t and_or(uint32_t y, uint32_t mask, uint32_t c) { return (y & mask) | c; }
__device__ __forceinline__ uint32_t opaque_u32(uint32_t x) {
  asm volatile("" : "+v"(x));
  return x;
}
// s_waitcnt immediate for vmcnt(0) alone (expcnt and lgkmcnt at their maxima)
constexpr int kWaitVm0 = 0x0F70;
__device__ __forceinline__ void wait_lgkm0() { asm volatile("s_waitcnt lgkmcnt(0)" : : : "memory"); }

template <int D, int GP, int KB, int VB, bool QJ, bool UN, class Setup>
__device__ void split_cached_chunk(const DArgs& a, int pr, int h_, int t0_, int t1_, const int32_t* s_blk,
                                   const uint2* s_pair, const u32x4* s_sgn, float* s_p, unsigned char* s_main,
                                   float* s_stat, bf16x8 (&A1)[D / 32][2], bf16x8 (&A3)[D / 32], const u32x4* s_A,
                                   const f32x4& ucst,
                                   float* m_out, float* l_out, int b, Setup&& setup) {
  using R = Rec<D, KB, VB, QJ>;
  constexpr int NS = ring_depth<D, GP, KB, VB, QJ, UN>();
  constexpr int NW = split_waves<D, GP, KB, VB, QJ, UN>();
  constexpr int KT = D / 32;
  constexpr int CS = D / 128;      // value column sets
  constexpr int RT = GP / 4;       // value row tiles per column set
  constexpr int CT = 8;            // value channel tiles per column set
  constexpr int QB = KB * D / 32;  // code bytes per lane quarter
  constexpr int QW = (QB + 3) / 4;
  constexpr int PPR = R::bytes / 16;          // 16-byte pieces per record
  constexpr int DPR = (PPR + 63) / 64;        // DMA instructions per record
  constexpr int DPS = 2 * DPR;                // DMA instructions per step
  static_assert((NS - 1) * DPS < 64, "vmcnt range");
  static_assert(PPR >= 64, "a record spans at least one full DMA window");
  // the wave index, KV head and token range are wave-uniform: saying so keeps
  // the step schedule below (ring slots, step indices, waits) and the record
  // addresses in scalar registers and scalar branches
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int h = __builtin_amdgcn_readfirstlane(h_);
  const int t0 = __builtin_amdgcn_readfirstlane(t0_), t1 = __builtin_amdgcn_readfirstlane(t1_);
  const int tok = lane & 15, kq = lane >> 4;
  const int64_t rec = a.rec[pr];
  // record (block, h) starts at head_base + block * blk_stride; the host
  // keeps num_kv_heads * record bytes below 2^31, so the product is one
  // 32 x 32 -> 64-bit multiply
  const uint64_t head_base = reinterpret_cast<uint64_t>(a.pool[pr]) + (uint64_t)h * (uint64_t)rec;
  const uint32_t blk_stride = (uint32_t)(a.Hkv * rec);
  float* sp = s_p + wave * SplitLds<D, GP, KB, VB, QJ, UN>::kPWave;
  unsigned char* ring = s_main + wave * NS * R::slot;
  const uint32_t ring_lds = lds_offset(ring);

  // per-lane byte offsets inside a record
  const int off_kc = R::kcodes + tok * (KB * D / 8) + kq * QB;
  const int off_kj = R::kqjl + tok * (D / 8) + kq * (D / 32);
  const int off_km = R::kmeta + tok * R::kmeta_slot;
  const int slot0 = (kq & 1) * 8;
  const int vhalf = kq >> 1;
  int off_vx[CS], off_vm[CS];
#pragma unroll
  for (int cs = 0; cs < CS; ++cs) {
    constexpr int WPS = VB == 4 ? 16 : 8;  // dword columns per column set
    const int wcol = cs * WPS + (VB == 4 ? (lane & 15) : (lane & 7));
    off_vx[cs] = vhalf * R::bytes + R::vcodes + (wcol * 16 + slot0) * 4;
    off_vm[cs] = vhalf * R::bytes + R::vmeta + ((4 * cs + ((lane & 15) >> 2)) * 16 + slot0) * 4;
  }

  // Stream the two records of step `st` into ring slot `sl`: record r's piece
  // k (16 bytes) lands at slot + r * bytes + 16 k; one DMA instruction per
  // window of 64 pieces, with the record base in SGPRs and a constant
  // per-lane offset.  The last window ends at the record's last piece and
  // overlaps the one before it (those pieces are written twice with the same
  // bytes), so every DMA runs on all 64 lanes and needs no lane mask.
  auto issue = [&](int st, int sl) {
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      const int blk = __builtin_amdgcn_readfirstlane(s_blk[2 * st + half]);
      const bool ok = blk >= 0;  // validated at staging
      const uint64_t base = head_base + (uint64_t)(uint32_t)(ok ? blk : 0) * blk_stride;
      const uint32_t dst = ring_lds + sl * R::slot + half * R::bytes;
#pragma unroll
      for (int j = 0; j < DPR; ++j) {
        const int p0 = j == DPR - 1 ? PPR - 64 : 64 * j;  // first piece of window j
        dma16(dst + 16 * p0, base, 16 * (p0 + lane));
      }
    }
  };

  f32x4 accv[CS][RT][CT];
#pragma unroll
  for (int cs = 0; cs < CS; ++cs)
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
#pragma unroll
      for (int ct = 0; ct < CT; ++ct) accv[cs][rt][ct] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
  float zacc[CS][RT];
#pragma unroll
  for (int cs = 0; cs < CS; ++cs)
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) zacc[cs][rt] = 0.f;
  float m_run[GP];
#pragma unroll
  for (int g = 0; g < GP; ++g) m_run[g] = -INFINITY;
  float lsum[4] = {0.f, 0.f, 0.f, 0.f};  // per-lane partial sums (rows of lanes 0..31)
  const uint32_t k4300 = UN ? opaque_u32(0x43004300u) : 0u;  // two bf16 128.0
  const int arow = lane & 15;
  // VB = 2: lane column j takes bytes 2 (j >> 3) and 2 (j >> 3) + 1 of its dword column
  uint32_t vsel[2];
#pragma unroll
  for (int bb = 0; bb < 2; ++bb) {
    const uint32_t by = 2u * (uint32_t)((lane & 15) >> 3) + (uint32_t)bb;
    vsel[bb] = by | ((4u + by) << 16);
  }

  auto compute = [&](const unsigned char* sb, int st) {
    // Issue priority: high through the score phase (LDS lookups feeding the
    // score MFMAs), normal for the value phase, so that the two waves of a
    // SIMD tend to be in different phases (measured ~1.5 % faster).
    __builtin_amdgcn_s_setprio(2);
    const int base = t0 + 32 * st;
    // block ids were validated at staging: -1 marks a block outside the pool
    const bool ok0 = __builtin_amdgcn_readfirstlane(s_blk[2 * st]) >= 0;
    const bool ok1 = __builtin_amdgcn_readfirstlane(s_blk[2 * st + 1]) >= 0;
    const bool full = ok0 && ok1 && base + 32 <= t1;  // every token of the step is live (uniform)
    // value codes and scales of the step, read first so that their LDS latency
    // hides under the score phase (the weight stores below could alias them)
    u32x4 vx0[CS], vx1[CS], vm0[CS], vm1[CS];
#pragma unroll
    for (int cs = 0; cs < CS; ++cs) {
      vx0[cs] = *reinterpret_cast<const u32x4*>(sb + off_vx[cs]);
      vx1[cs] = *reinterpret_cast<const u32x4*>(sb + off_vx[cs] + 16);
      vm0[cs] = *reinterpret_cast<const u32x4*>(sb + off_vm[cs]);
      vm1[cs] = *reinterpret_cast<const u32x4*>(sb + off_vm[cs] + 16);
    }
    // ------------------------------------------------------------ scores
    // v[half][r]: MFMA output row 4 (lane / 16) + r of the half's 16 tokens
    // (column = token); rows 0..GP-1 carry the hi parts of the heads, rows
    // GP..2GP-1 the lo parts.
    float v[2][4];
    // k-slice outer, record inner: only one slice's A operands are live
    f32x4 am[2], aq[2];
    uint32_t cw[2][QW + 1], kj[2][D / 128], km[2];
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      const unsigned char* hb = sb + half * R::bytes;
      // equally spaced codebook: the accumulator starts at the rows' offset
      // constant (see the arithmetic operands below)
      am[half] = UN ? ucst : f32x4{0.f, 0.f, 0.f, 0.f};
      aq[half] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int i = 0; i < QW; ++i) cw[half][i] = *reinterpret_cast<const uint32_t*>(hb + off_kc + 4 * i);
      cw[half][QW] = 0;
      if constexpr (QJ) {
#pragma unroll
        for (int i = 0; i < D / 128; ++i) kj[half][i] = *reinterpret_cast<const uint32_t*>(hb + off_kj + 4 * i);
      }
      km[half] = QJ ? *reinterpret_cast<const uint32_t*>(hb + off_km)
                    : (uint32_t)*reinterpret_cast<const uint16_t*>(hb + off_km);
    }
#pragma unroll
    for (int kt = 0; kt < KT; ++kt) {
      bf16x8 a1[2], a3;
      if constexpr (lds_a<D, GP, KB, VB, QJ, UN>()) {
        a1[0] = __builtin_bit_cast(bf16x8, s_A[(3 * kt) * 64 + lane]);
        a1[1] = __builtin_bit_cast(bf16x8, s_A[(3 * kt + 1) * 64 + lane]);
        if constexpr (QJ) a3 = __builtin_bit_cast(bf16x8, s_A[(3 * kt + 2) * 64 + lane]);
      } else {
        a1[0] = A1[kt][0];
        a1[1] = A1[kt][1];
        a3 = A3[kt];
      }
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        constexpr int TB = 8 * KB;
        const int bp = kt * TB;
        const uint32_t win = bp % 32 == 0 ? cw[half][bp / 32]
                                          : __builtin_amdgcn_alignbit(cw[half][bp / 32 + 1], cw[half][bp / 32], bp % 32);
        if constexpr (KB == 8) {
          // 8-bit codes: one lookup per code in the one-code table (bf16 hi
          // | lo << 16 of c[idx]), so MFMA m takes coordinates 4m .. 4m+3 as
          // {hi, lo} pairs (the A operand repeats each coordinate twice)
          const uint32_t* s_one = reinterpret_cast<const uint32_t*>(s_pair);
#pragma unroll
          for (int m = 0; m < 2; ++m) {
            const uint32_t cb = cw[half][2 * kt + m];
            const u32x4 b = {s_one[cb & 0xFFu], s_one[(cb >> 8) & 0xFFu], s_one[(cb >> 16) & 0xFFu], s_one[cb >> 24]};
            am[half] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a1[m], __builtin_bit_cast(bf16x8, b), am[half], 0, 0, 0);
          }
        } else if constexpr (UN) {
          // c[idx] = c0 + step idx needs no table: B element = bf16 of
          // 128 + idx (0x4300 | idx, exact), built from the code bits alone.
          // Dword j holds codes j and j + 4 of the slice: y has codes 0-3 in
          // its low half and codes 4-7 in its high half, so one shift and one
          // and-or place both.
          constexpr uint32_t m4 = (1u << (4 * KB)) - 1u;
          const uint32_t y = (win & m4) | ((win << (16 - 4 * KB)) & (m4 << 16));
          constexpr uint32_t m2 = ((1u << KB) - 1u) * 0x00010001u;
          u32x4 bu;
#pragma unroll
          for (int j = 0; j < 4; ++j) bu[j] = and_or(y >> (KB * j), m2, k4300);
          am[half] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a1[0], __builtin_bit_cast(bf16x8, bu), am[half], 0, 0, 0);
        } else {
          // pair entries {hi, lo}: MFMA m takes pairs 2m, 2m+1 (coordinates 4m .. 4m+3)
          uint2 pe[4];
#pragma unroll
          for (int pi = 0; pi < 4; ++pi) pe[pi] = s_pair[(win >> (2 * KB * pi)) & ((1u << (2 * KB)) - 1u)];
          const u32x4 b0 = {pe[0].x, pe[0].y, pe[1].x, pe[1].y};
          const u32x4 b1 = {pe[2].x, pe[2].y, pe[3].x, pe[3].y};
          am[half] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a1[0], __builtin_bit_cast(bf16x8, b0), am[half], 0, 0, 0);
          am[half] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a1[1], __builtin_bit_cast(bf16x8, b1), am[half], 0, 0, 0);
        }
        if constexpr (QJ) {
          const u32x4 bq = s_sgn[(kj[half][kt / 4] >> (8 * (kt % 4))) & 0xFFu];
          aq[half] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a3, __builtin_bit_cast(bf16x8, bq), aq[half], 0, 0, 0);
        }
      }
    }
    // logit = log2(e) sm_scale n (q~.c + kappa gamma p.sign), with
    // log2(e) sm_scale folded into q~ and kappa log2(e) sm_scale into p (the
    // A operands)
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      const float n = f16_bits_to_f32((uint16_t)(km[half] & 0xFFFFu));
      if constexpr (QJ) {
        const float nk = n * f16_bits_to_f32((uint16_t)(km[half] >> 16));
#pragma unroll
        for (int r = 0; r < 4; ++r) v[half][r] = __builtin_fmaf(nk, aq[half][r], n * am[half][r]);
      } else {
#pragma unroll
        for (int r = 0; r < 4; ++r) v[half][r] = n * am[half][r];
      }
    }
    // x[r]: hi + lo of head row r, one swap per row.  GP = 4: the hi and lo
    // rows sit 16 lanes apart; after the swap lanes 0-15 hold the first 16
    // tokens, lanes 16-31 the second 16 (lanes 32-63 hold zero rows and are
    // never read back).  GP = 8: rows 32 lanes apart; lanes 0-31 take the
    // first 16 tokens (heads 0-3 | 4-7 by lane bit 4), lanes 32-63 the second.
    const int sh = GP == 4 ? ((lane >> 4) & 1) : (lane >> 5);
    float x[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      auto sw = GP == 4 ? __builtin_amdgcn_permlane16_swap(__float_as_uint(v[0][r]), __float_as_uint(v[1][r]), false, false)
                        : __builtin_amdgcn_permlane32_swap(__float_as_uint(v[0][r]), __float_as_uint(v[1][r]), false, false);
      x[r] = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
    }
    const int my_tok = base + 16 * sh + tok;
    if (!full) {  // uniform: dead tokens of a partial step get -inf
      const bool live = (sh ? ok1 : ok0) && my_tok < t1;
#pragma unroll
      for (int r = 0; r < 4; ++r) x[r] = live ? x[r] : -INFINITY;
    }
    if (a.scores) {  // uniform: estimated q.k of the live tokens
      const int ln = (int)opaque_u32((uint32_t)lane);  // recomputed here, not kept live across the loop
      const int hh0 = GP == 8 && (ln & 16) ? 4 : 0;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        if ((GP == 8 || ln < 32) && hh0 + r < a.G && x[r] != -INFINITY)
          a.scores[((int64_t)b * a.Hq + h * a.G + hh0 + r) * a.scores_stride + my_tok] = x[r] * a.inv_logit_scale;
      }
    }
    // ------------------------------------------------------------ softmax
    // Each lane holds four distinct (head, token) logits (see x above).  The
    // block maxima are only needed when some logit passes its head's
    // reference by more than kLazyMax: that test is one compare per logit
    // and a ballot; the maxima are formed inside the (rare) rescale branch.
    bool grow;
    {
      const int ln = (int)opaque_u32((uint32_t)lane);
      const bool hi = GP == 8 && (ln & 16);  // GP = 8: lanes 16-31 / 48-63 carry heads 4..7
      uint64_t over = 0;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float lim = (hi ? m_run[(4 + r) % GP] : m_run[r]) + kLazyMax;
        over |= __builtin_amdgcn_ballot_w64(x[r] > lim);
      }
      if constexpr (GP == 4) over &= 0xFFFFFFFFull;  // lanes 32-63 hold no logits
      grow = over != 0;
    }
    if (grow) {  // uniform: some head's block max passed its reference; rescale what was accumulated
      const int ln = (int)opaque_u32((uint32_t)lane);  // lane predicates are formed here, not kept live
      // block maxima: 16-lane row maxima, then the rows holding each head
      float y0 = x[0], y1 = x[1], y2 = x[2], y3 = x[3];
      row_max16x4(y0, y1, y2, y3);
      const float ys[4] = {y0, y1, y2, y3};
      float mt[GP];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int yr = __float_as_int(ys[r]);
        if constexpr (GP == 4) {
          mt[r] = fmaxf(__int_as_float(__builtin_amdgcn_readlane(yr, 0)), __int_as_float(__builtin_amdgcn_readlane(yr, 16)));
        } else {
          mt[r] = fmaxf(__int_as_float(__builtin_amdgcn_readlane(yr, 0)), __int_as_float(__builtin_amdgcn_readlane(yr, 32)));
          mt[4 + r] = fmaxf(__int_as_float(__builtin_amdgcn_readlane(yr, 16)), __int_as_float(__builtin_amdgcn_readlane(yr, 48)));
        }
      }
      float alpha[GP];
#pragma unroll
      for (int g = 0; g < GP; ++g) {
        const float mn = fmaxf(m_run[g], mt[g]);
        alpha[g] = __builtin_amdgcn_exp2f(m_run[g] - mn);  // 0 while m_run is -inf, 1 if unchanged
        m_run[g] = mn;
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) lsum[r] *= (GP == 8 && (ln & 16)) ? alpha[(4 + r) % GP] : alpha[r];
#pragma unroll
      for (int cs = 0; cs < CS; ++cs)
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
#pragma unroll
          for (int r = 0; r < 4; ++r) {
#pragma unroll
            for (int ct = 0; ct < CT; ++ct) accv[cs][rt][ct][r] *= alpha[4 * rt + r];
          }
          float az = alpha[4 * rt];
#pragma unroll
          for (int r = 1; r < 4; ++r) az = ((ln & 3) == r) ? alpha[4 * rt + r] : az;
          zacc[cs][rt] *= az;
        }
    }
    {
      // weight of (head hh0 + r, token tokw); with GP = 4 lanes 32-63 write
      // the unread second copy (address arithmetic instead of a lane mask)
      const int ln = (int)opaque_u32((uint32_t)lane);
      const int hh0 = GP == 8 ? ((ln >> 4) & 1) * 4 : 0;
      float* spw = sp + (ln & 15) + 16 * sh + (GP == 4 ? (ln >> 5) * (GP * 32) : 0);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float mr = (GP == 8 && hh0) ? m_run[(4 + r) % GP] : m_run[r];
        const float p = __builtin_amdgcn_exp2f(x[r] - (mr == -INFINITY ? 0.f : mr + kLazyMax));
        lsum[r] += p;
        spw[(hh0 + r) * 32] = p;
      }
    }
    wait_lgkm0();  // the weights are in LDS
    __builtin_amdgcn_s_setprio(0);
    // ------------------------------------------------------------ values
    // fp16 MFMA: A = p s as fp16 hi + lo, B = the code bits placed in the
    // mantissa of a zero exponent: a code at bits k .. k + b - 1 is the fp16
    // subnormal q 2^(k - 24), exact, with no offset to subtract (sigma = 2^k
    // is divided out per column at the end), so B costs one shift and / or
    // one AND per dword.  The codes sit at bit 4 or above: the matrix cores
    // take subnormal operands, but products with the smallest ones (codes in
    // bits 0..3) measured ~8x less precise per product than with codes at
    // bits 4..7, which are as precise as normal operands.
    const bool vblk_ok = vhalf ? ok1 : ok0;
    const int vtok0 = base + 8 * kq;
#pragma unroll
    for (int cs = 0; cs < CS; ++cs) {
      const u32x4 x0 = vx0[cs], x1 = vx1[cs], m0 = vm0[cs], m1 = vm1[cs];
      const uint32_t xv[8] = {x0[0], x0[1], x0[2], x0[3], x1[0], x1[1], x1[2], x1[3]};
      uint32_t sz[8] = {m0[0], m0[1], m0[2], m0[3], m1[0], m1[1], m1[2], m1[3]};
      if (!full) {
#pragma unroll
        for (int e = 0; e < 8; ++e) sz[e] = (vblk_ok && (vtok0 + e) < t1) ? sz[e] : 0u;
      }
      // B tiles: byte-gather two tokens' code bytes into the halves of a dword
      u32x4 bv[CT];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if constexpr (VB == 4) {
#pragma unroll
          for (int bi = 0; bi < 4; ++bi) {
            const uint32_t y = __builtin_amdgcn_perm(xv[2 * i + 1], xv[2 * i], (uint32_t)bi | ((uint32_t)(4 + bi) << 16));
            bv[2 * bi][i] = (y << 4) & 0x00F000F0u;
            bv[2 * bi + 1][i] = y & 0x00F000F0u;
          }
        } else {
#pragma unroll
          for (int bb = 0; bb < 2; ++bb) {
            const uint32_t y = __builtin_amdgcn_perm(xv[2 * i + 1], xv[2 * i], vsel[bb]);
            bv[4 * bb + 0][i] = (y << 4) & 0x00300030u;
            bv[4 * bb + 1][i] = (y << 4) & 0x00C000C0u;
            bv[4 * bb + 2][i] = y & 0x00300030u;
            bv[4 * bb + 3][i] = y & 0x00C000C0u;
          }
        }
      }
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) {
        const int hd = 4 * rt + (arow & 3);
        const f32x4 pa = *reinterpret_cast<const f32x4*>(sp + hd * 32 + 8 * kq);
        const f32x4 pb = *reinterpret_cast<const f32x4*>(sp + hd * 32 + 8 * kq + 4);
        const float pw[8] = {pa[0], pa[1], pa[2], pa[3], pb[0], pb[1], pb[2], pb[3]};
        f16x8 Ah, Al;
        float z = zacc[cs][rt];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float sv = f16_bits_to_f32((uint16_t)(sz[e] & 0xFFFFu));
          const _Float16 hv = (_Float16)__builtin_fmaf(pw[e], sv, 0.f);
          Ah[e] = hv;
          Al[e] = (_Float16)__builtin_fmaf(pw[e], sv, -(float)hv);
          z = __builtin_fmaf(pw[e], f16_bits_to_f32((uint16_t)(sz[e] >> 16)), z);
        }
        zacc[cs][rt] = z;
#pragma unroll
        for (int ct = 0; ct < CT; ++ct) {
          const f16x8 B = __builtin_bit_cast(f16x8, bv[ct]);
          accv[cs][rt][ct] = __builtin_amdgcn_mfma_f32_16x16x32_f16(Ah, B, accv[cs][rt][ct], 0, 0, 0);
          accv[cs][rt][ct] = __builtin_amdgcn_mfma_f32_16x16x32_f16(Al, B, accv[cs][rt][ct], 0, 0, 0);
        }
      }
    }
  };

  // ---- the stream.  Wave w takes steps w, w + NW, w + 2 NW, ... in order,
  // from a scalar counter: every call sums the same steps in the same order,
  // so outputs and scores are bit-identical from run to run and between eager
  // and graph-replayed launches.  (A schedule in which each wave claimed the
  // next free step from an LDS counter measured no faster on the decode
  // workload and ~2 % slower on the long and ragged ones: the claim's atomic
  // and its wait sat on every step's critical path.)  Ring depth NS;
  // stq[k] is the step held by slot k (-1: none).
  const int nsteps = (t1 - t0 + 31) / 32;
  const bool exact_wait = a.scores == nullptr;  // score stores also count in vmcnt
  bool more = true;
  int nxt = NW * (NS - 1) + wave;
  auto next_step = [&](int) -> int {
    if (!more) return -1;
    const int v = nxt;
    nxt += NW;
    more = v < nsteps;
    return more ? v : -1;
  };
  int stq[NS];
#pragma unroll
  for (int k = 0; k < NS - 1; ++k) {  // the first steps of each wave are fixed: wave + NW k
    stq[k] = wave + NW * k < nsteps ? wave + NW * k : -1;
    if (stq[k] >= 0) issue(stq[k], k);
  }
  more = stq[NS - 2] >= 0;
  stq[NS - 1] = -1;
  setup(A1, A3);  // per-item work that needs no cache data runs while the first steps stream in
  // one ring lap per outer iteration, so every slot offset is a constant
  auto stream_step = [&](auto slot_c) -> bool {
    constexpr int SL = decltype(slot_c)::value;
    constexpr int FREE = (SL + NS - 1) % NS;  // the slot of the step computed last
    if (stq[SL] < 0) return false;
    stq[FREE] = next_step(stq[SL]);
    if (stq[FREE] >= 0) {
      wait_lgkm0();  // ring slot reuse: the reads of the step that used it are complete
      issue(stq[FREE], FREE);
    }
    int ahead = 0;  // steps issued after this one (the slots after SL in ring order)
#pragma unroll
    for (int k = 1; k < NS; ++k) ahead += stq[(SL + k) % NS] >= 0 ? 1 : 0;
    if (!exact_wait || ahead == 0)
      wait_vmcnt<0>();
    else if (ahead == 1)
      wait_vmcnt<DPS>();
    else
      wait_vmcnt<(NS - 1) * DPS>();
    compute(ring + SL * R::slot, stq[SL]);
    return true;
  };
  for (;;) {
    if (!stream_step(std::integral_constant<int, 0>{})) break;
    if (!stream_step(std::integral_constant<int, 1>{})) break;
    if constexpr (NS == 3)
      if (!stream_step(std::integral_constant<int, 2>{})) break;
  }
  wait_vmcnt<0>();
  __syncthreads();  // every wave is done with the ring before it becomes the merge area

  // ---------------------------------------------------------------- merge
  float* s_merge = reinterpret_cast<float*>(s_main);
  // zacc: sum the four token quarters (lanes l, l^16, l^32, l^48)
#pragma unroll
  for (int cs = 0; cs < CS; ++cs)
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) zacc[cs][rt] = lane_swap16_sum(lane_swap32_sum(zacc[cs][rt]));
  float* mw = s_merge + wave * GP * D;
  // each wave writes its own un-normalised acc[head][channel]: output row
  // (group lane/16, head 4 rt + r) of column j is kept where the column's
  // channel belongs to that group
  const int j = lane & 15, gl = lane >> 4;
#pragma unroll
  for (int cs = 0; cs < CS; ++cs)
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        // zero-point term of row (group gl, head 4 rt + r) sits in A row 4 gl + r
        const float zv = __shfl(zacc[cs][rt], 4 * gl + r, 64);
#pragma unroll
        for (int ct = 0; ct < CT; ++ct) {
          int ch;
          float inv;  // 2^24 / sigma of the tile's field position
          if constexpr (VB == 4) {
            ch = 128 * cs + 8 * j + 2 * (ct >> 1) + (ct & 1);
            inv = 1048576.f;
          } else {
            ch = 128 * cs + 16 * (j & 7) + 4 * (2 * (j >> 3) + (ct >> 2)) + (ct & 3);
            // 2-bit fields at bits 4 and 6: sigma 16 and 64
            inv = (ct & 1) ? 262144.f : 1048576.f;
          }
          if ((ch >> 5) - 4 * cs == gl)
            mw[(4 * rt + r) * D + ch] = __builtin_fmaf(accv[cs][rt][ct][r], inv, zv);
        }
      }
  // l per head: row sums of the lane groups that held the head's two token halves
  float lh[GP];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int lw = __float_as_int(row_sum16(lsum[r]));
    if constexpr (GP == 4) {
      lh[r] = __int_as_float(__builtin_amdgcn_readlane(lw, 0)) + __int_as_float(__builtin_amdgcn_readlane(lw, 16));
    } else {
      lh[r] = __int_as_float(__builtin_amdgcn_readlane(lw, 0)) + __int_as_float(__builtin_amdgcn_readlane(lw, 32));
      lh[4 + r] = __int_as_float(__builtin_amdgcn_readlane(lw, 16)) + __int_as_float(__builtin_amdgcn_readlane(lw, 48));
    }
  }
  if (lane == 0) {
#pragma unroll
    for (int g = 0; g < GP; ++g) {
      s_stat[(wave * GP + g) * 2] = m_run[g] + kLazyMax;  // the weights' effective reference
      s_stat[(wave * GP + g) * 2 + 1] = lh[g];
    }
  }
  __syncthreads();
  // combine the four waves; results for head g in m_out[g], l_out[g] and s_merge[g][:]
  const int tid = threadIdx.x;
  for (int idx = tid; idx < GP * D; idx += NW * 64) {
    const int g = idx / D;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < NW; ++w) M = fmaxf(M, s_stat[(w * GP + g) * 2]);
    float acc = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      const float lwv = s_stat[(w * GP + g) * 2 + 1];
      const float f = lwv > 0.f ? __builtin_amdgcn_exp2f(s_stat[(w * GP + g) * 2] - M) : 0.f;
      acc += f * s_merge[w * GP * D + idx];
    }
    s_merge[idx] = acc;  // each idx is read and written by this thread only
  }
  if (tid < GP) {
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < NW; ++w) M = fmaxf(M, s_stat[(w * GP + tid) * 2]);
    float L = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      const float lwv = s_stat[(w * GP + tid) * 2 + 1];
      L += lwv > 0.f ? lwv * __builtin_amdgcn_exp2f(s_stat[(w * GP + tid) * 2] - M) : 0.f;
    }
    m_out[tid] = L > 0.f ? M : -INFINITY;
    l_out[tid] = L;
  }
  __syncthreads();
}

// Recent full-precision window: exact scores <q, k> with the unrotated query
// and bf16 keys, bf16 values.  One head at a time (few registers, so the
// streaming path's allocation is unaffected); wave w takes tokens w, w + NW,
// ...: its 64 lanes read a token's key row (and later its value row), d/64
// channels each, so every row is one coalesced read, and the dot products
// are wave reductions.  The softmax runs per head over the window; the
// waves' partial value sums are added in LDS in wave order (deterministic).
template <int D, int GP, int NW>
__device__ void split_recent(const DArgs& a, int b, int h, int R, float* s_p, float* s_merge, float* m_out,
                             float* l_out) {
  constexpr int P = D / 64;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const uint16_t* kb = a.rk + (((int64_t)b * a.Hkv + h) * a.W) * D;
  const uint16_t* vb = a.rv + (((int64_t)b * a.Hkv + h) * a.W) * D;
  float* lg = s_merge;                  // [GP][R] logits, then weights; R <= W
  float* part = s_merge + GP * a.W;     // [GP][D] value sums, added wave by wave
  const int64_t q0 = ((int64_t)b * a.Hq + (int64_t)h * a.G) * D;
  auto load_row = [&](const uint16_t* row, float (&x)[P]) {
    if constexpr (P == 2) {
      const uint32_t w = *reinterpret_cast<const uint32_t*>(row + 2 * lane);
      x[0] = __uint_as_float(w << 16);
      x[1] = __uint_as_float(w & 0xFFFF0000u);
    } else {
      const uint2 w = *reinterpret_cast<const uint2*>(row + 4 * lane);
      x[0] = __uint_as_float(w.x << 16);
      x[1] = __uint_as_float(w.x & 0xFFFF0000u);
      x[2] = __uint_as_float(w.y << 16);
      x[3] = __uint_as_float(w.y & 0xFFFF0000u);
    }
  };
  const int Lc = seq_cached(a, b);
#pragma unroll 1
  for (int g = 0; g < a.G; ++g) {
    float qv[P];
#pragma unroll
    for (int e = 0; e < P; ++e) {
      const int64_t i = q0 + (int64_t)g * D + P * lane + e;
      qv[e] = a.q_bf16 ? bf16_to_f32(reinterpret_cast<const uint16_t*>(a.q)[i]) : reinterpret_cast<const float*>(a.q)[i];
    }
#pragma unroll 1
    for (int t = wave; t < R; t += NW) {
      float kx[P];
      load_row(kb + (int64_t)t * D, kx);
      float sdot = 0.f;
#pragma unroll
      for (int e = 0; e < P; ++e) sdot = __builtin_fmaf(qv[e], kx[e], sdot);
      sdot = wave_sum_xl(sdot);
      if (lane == 0) {
        lg[g * R + t] = sdot * a.logit_scale;
        if (a.scores) a.scores[((int64_t)b * a.Hq + h * a.G + g) * a.scores_stride + Lc + t] = sdot;
      }
    }
  }
  __syncthreads();
  if (tid < a.G) {
    float M = -INFINITY;
    for (int t = 0; t < R; ++t) M = fmaxf(M, lg[tid * R + t]);
    float L = 0.f;
    for (int t = 0; t < R; ++t) {
      const float p = __builtin_amdgcn_exp2f(lg[tid * R + t] - M);
      lg[tid * R + t] = p;
      L += p;
    }
    m_out[tid] = M;
    l_out[tid] = L;
  }
  __syncthreads();
#pragma unroll 1
  for (int g = 0; g < a.G; ++g) {
    float acc[P];
#pragma unroll
    for (int e = 0; e < P; ++e) acc[e] = 0.f;
#pragma unroll 1
    for (int t = wave; t < R; t += NW) {
      float vx[P];
      load_row(vb + (int64_t)t * D, vx);
      const float w = lg[g * R + t];
#pragma unroll
      for (int e = 0; e < P; ++e) acc[e] = __builtin_fmaf(w, vx[e], acc[e]);
    }
#pragma unroll 1
    for (int w = 0; w < NW; ++w) {
      if (wave == w) {
#pragma unroll
        for (int e = 0; e < P; ++e) {
          float* pp = part + g * D + P * lane + e;
          *pp = (w == 0 ? 0.f : *pp) + acc[e];
        }
      }
      __syncthreads();
    }
  }
  // move the sums to s_merge[g][c] (they may overlap the part area when
  // the window is shorter than d: read all, then write)
  constexpr int NR = (GP * D + NW * 64 - 1) / (NW * 64);
  float res[NR];
#pragma unroll
  for (int r = 0; r < NR; ++r) {
    const int idx = tid + r * NW * 64;
    res[r] = idx < a.G * D ? part[idx] : 0.f;
  }
  __syncthreads();
#pragma unroll
  for (int r = 0; r < NR; ++r) {
    const int idx = tid + r * NW * 64;
    if (idx < a.G * D) s_merge[idx] = res[r];
  }
  __syncthreads();
}

// q~ = D2 H D1 q / sqrt(d) of the G query heads of (b, h) into s_q (wave w
// rotates heads w, w + 4 in registers: butterflies within a lane for the low
// index bits, shuffles for the others), then p = S q~ on the matrix cores into
// s_pq: A rows = heads (fp16 hi/lo of q~ 2^-e_g, with 2^e_g above the head's
// largest |q~_j| so fp16 cannot overflow), B = the 16 S tiles of the context,
// three products per tile; wave w takes column tiles w, w + NW, ...
template <int D, int NW, bool QJ>
__device__ __forceinline__ void rotate_project(const DArgs& a, const DevTables& dv, int b, int h, float* s_q, float* s_pq,
                               int* s_exp) {
  constexpr int P = D / 64;
  constexpr int KT = D / 32, NT = D / 16, NTW = (NT + NW - 1) / NW;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int G = a.G;
  const int64_t q0 = ((int64_t)b * a.Hq + (int64_t)h * G) * D;
  // the S tiles do not depend on q: load them first (MSE-only keys need no p)
  f16x8 bhi[NTW][KT], blo[NTW][KT];
#pragma unroll
  for (int i = 0; i < (QJ ? NTW : 0); ++i) {
#pragma unroll
    for (int kt = 0; kt < KT; ++kt) {
      const int ntc = wave + NW * i < NT ? wave + NW * i : 0;  // waves past the last tile read tile 0, unused
      const size_t tb = ((((size_t)ntc) * KT + kt) * 2) * 64 * 8;
      bhi[i][kt] = *reinterpret_cast<const f16x8*>(dv.s_tiles + tb + lane * 8);
      blo[i][kt] = *reinterpret_cast<const f16x8*>(dv.s_tiles + tb + 512 + lane * 8);
    }
  }
  for (int g = wave; g < G; g += NW) {
    float x[P];
#pragma unroll
    for (int e = 0; e < P; ++e) {
      const int j = P * lane + e;
      const float v = a.q_bf16 ? bf16_to_f32(reinterpret_cast<const uint16_t*>(a.q)[q0 + g * D + j])
                               : reinterpret_cast<const float*>(a.q)[q0 + g * D + j];
      x[e] = v * dv.signs1[j];
    }
#pragma unroll
    for (int hs = 1; hs < P; hs <<= 1) {
#pragma unroll
      for (int e = 0; e < P; ++e) {
        if ((e & hs) == 0) {
          const float p = x[e], q = x[e + hs];
          x[e] = p + q;
          x[e + hs] = p - q;
        }
      }
    }
    {
      const float s1 = lane_sign<1>(lane), s2 = lane_sign<2>(lane), s4 = lane_sign<4>(lane);
      const float s8 = lane_sign<8>(lane), s16 = lane_sign<16>(lane), s32 = lane_sign<32>(lane);
#pragma unroll
      for (int e = 0; e < P; ++e) {
        float v = x[e];
        v = wht_xlane<1>(v, s1);
        v = wht_xlane<2>(v, s2);
        v = wht_xlane<4>(v, s4);
        v = wht_xlane<8>(v, s8);
        v = wht_xlane<16>(v, s16);
        x[e] = wht_xlane<32>(v, s32);
      }
    }
    const float inv = 1.0f / __builtin_sqrtf((float)D);
    float amax = 0.f;
#pragma unroll
    for (int e = 0; e < P; ++e) {
      const int j = P * lane + e;
      const float v = x[e] * inv * dv.signs2[j];
      s_q[g * D + j] = v;
      amax = fmaxf(amax, fabsf(v));
    }
    amax = wave_max_xl(amax);
    if (lane == 0) s_exp[g] = amax > 0.f ? (int)((__float_as_uint(amax) >> 23) & 0xFFu) - 126 : 0;
  }
  __syncthreads();
  if constexpr (!QJ) return;
  const int arow = lane & 15, kq = lane >> 4;
  // rows >= G read row 0 (unconditional vector reads) and are zeroed by the scale
  const int arow_c = arow < G ? arow : 0;
  const float ascale = arow < G ? __builtin_ldexpf(1.0f, -s_exp[arow_c]) : 0.f;
  f16x8 ahi[KT], alo[KT];
#pragma unroll
  for (int kt = 0; kt < KT; ++kt) {
    const f32x4 qa = *reinterpret_cast<const f32x4*>(s_q + arow_c * D + 32 * kt + 8 * kq);
    const f32x4 qb = *reinterpret_cast<const f32x4*>(s_q + arow_c * D + 32 * kt + 8 * kq + 4);
    const float qs[8] = {qa[0], qa[1], qa[2], qa[3], qb[0], qb[1], qb[2], qb[3]};
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float v = qs[e] * ascale;
      const _Float16 hv = (_Float16)v;
      ahi[kt][e] = hv;
      alo[kt][e] = (_Float16)(v - (float)hv);
    }
  }
  const float unscale = 1.0f / (float)(1 << kSScaleLog2);
#pragma unroll
  for (int i = 0; i < NTW; ++i) {
    const int nt = wave + NW * i;
    if (nt >= NT) break;  // uniform
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kt = 0; kt < KT; ++kt) {
      acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(ahi[kt], bhi[i][kt], acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(ahi[kt], blo[i][kt], acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(alo[kt], bhi[i][kt], acc, 0, 0, 0);
    }
    // result row 4 (lane / 16) + r (a head), column lane % 16
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int g = 4 * kq + r;
      if (g < G) s_pq[g * D + 16 * nt + arow] = __builtin_ldexpf(acc[r] * unscale, s_exp[g]);
    }
  }
  __syncthreads();
}

// One workgroup of four waves per work item (b, h, c): chunk c of the cached
// tokens of (sequence b, KV head h), or the recent window when c is the last
// split.  The items of this preset are enumerated in (b, h, c) order by a scan
// every workgroup runs at start-up; workgroup w takes the contiguous range
// [w total / grid, (w + 1) total / grid), so consecutive items mostly share
// (b, h) and reuse its rotated query operands.
// UN: the preset's codebook is equally spaced (c_k = c0 + k step) and the
// score takes c[idx] arithmetically instead of from the pair table.
template <int D, int GP, int KB, int VB, bool QJ, bool UN>
__global__ __launch_bounds__((split_waves<D, GP, KB, VB, QJ, UN>() * 64)) void decode_split_kernel(DArgs a, int pr) {
  constexpr int NW = split_waves<D, GP, KB, VB, QJ, UN>();
  constexpr int KT = D / 32;
  extern __shared__ __attribute__((aligned(16))) unsigned char lds[];
  using SL = SplitLds<D, GP, KB, VB, QJ, UN>;
  float* s_p = reinterpret_cast<float*>(lds);
  float* s_stat = s_p + NW * SL::kPWave;
  int32_t* s_blk = reinterpret_cast<int32_t*>(s_stat + NW * GP * 2);
  unsigned char* s_main = lds + SL::kMainOffset;
  float* s_merge = reinterpret_cast<float*>(s_main);
  u32x4* s_A = reinterpret_cast<u32x4*>(lds + SL::kPBytes + SL::kStatBytes + SL::kBlkBytes);
  __shared__ uint2 s_pair[256];  // centroid pair -> {bf16 hi parts, bf16 lo parts}
  __shared__ u32x4 s_sgn[QJ ? 256 : 1];  // sign byte -> 8 bf16 of +-1 (bit i -> element i)
  __shared__ float s_m[kMaxG], s_l[kMaxG];
  __shared__ __attribute__((aligned(16))) float s_q[GP * D];
  __shared__ __attribute__((aligned(16))) float s_pq[GP * D];
  __shared__ int s_exp[GP];
  const int tid = threadIdx.x, lane = tid & 63;

  // tables: centroid pairs of this preset, +-1 patterns of sign bytes
  const DevTables& dv = a.dev[pr];
  static_assert(KB == 8 || (1 << (2 * KB)) <= NW * 64, "one centroid pair per thread");
  static_assert(KB != 8 || 256 <= NW * 64, "one code-table entry per thread");
  // entries of the score table: two-code pairs (2-4-bit keys), or single codes
  // (8-bit keys, stored in the same LDS as dwords)
  constexpr int kTab = KB == 8 ? 256 : (1 << (2 * KB));
  // loaded here, stored after the scan's first loads are issued, so the two
  // global round trips overlap
  const uint2 pair_v = KB == 8 ? make_uint2(tid < 256 ? dv.code_lut[tid] : 0u, 0u)
                      : !UN && tid < kTab ? make_uint2(dv.pair_lut[2 * tid], dv.pair_lut[2 * tid + 1])
                                                     : make_uint2(0u, 0u);
  {
    u32x4 w;
#pragma unroll
    for (int e = 0; e < 4; ++e)
      w[e] = (((tid >> (2 * e)) & 1) ? 0x3F80u : 0xBF80u) | ((((tid >> (2 * e + 1)) & 1) ? 0x3F80u : 0xBF80u) << 16);
    if (QJ && tid < 256) s_sgn[tid] = w;  // one entry per thread
  }

  auto store_table = [&](int t) {
    if constexpr (KB == 8) {
      if (t < 256) reinterpret_cast<uint32_t*>(s_pair)[t] = pair_v.x;
    } else if (!UN && t < kTab) {
      s_pair[t] = pair_v;
    }
  };

  bf16x8 A1[KT][2], A3[KT];
  f32x4 ucst = {0.f, 0.f, 0.f, 0.f};  // equally spaced codebook: score rows' offsets
  int ready_bh = -1;  // (b, h) whose query operands A1 / A3 / ucst hold

  // One item: split c of KV head h of sequence b, which has Lc cached tokens.
  // kDirect: at most one split per sequence (the output is written here).
  auto run_item = [&](int b, int h, int c, int Lc, auto direct_c) {
    constexpr bool kDirect = decltype(direct_c)::value;
    using R = Rec<D, KB, VB, QJ>;
    constexpr bool kEarlyRotate = D == 128;
    constexpr int kStageRounds = (kMaxChunk / 16 + 2 + NW * 64 - 1) / (NW * 64);
    const int nq_chunks = (Lc + a.chunk - 1) / a.chunk;
    const bool cached = c < nq_chunks;  // uniform
    const int t0 = c * a.chunk;
    const int t1 = min(t0 + a.chunk, Lc);
    const int bh = b * a.Hkv + h;
    // One load phase per item: the chunk's block ids go to registers (read
    // up to the end of the table row, masked past the chunk's end once the
    // length is known), then (d = 128) the query rotation / projection of a
    // new (b, h) issues its own loads, so the round trips overlap and all of
    // it completes before the first cache step is requested.  In direct mode
    // none of it waits for the sequence length.  With d = 256 the projection
    // tiles take too many registers to share the phase; the rotation then
    // runs after the first steps are requested.
    if (kDirect || cached) {
      const int nstage = (a.chunk >> 4) + 2;
      const int row_left = a.max_blocks - (t0 >> 4);
      const int32_t* btrow = a.bt + (int64_t)b * a.max_blocks + (t0 >> 4);
      const int64_t pblocks = a.pool_blocks[pr];
      int blk[kStageRounds];
#pragma unroll
      for (int r = 0; r < kStageRounds; ++r) {
        const int i = tid + r * NW * 64;
        blk[r] = (i < nstage && i < row_left) ? btrow[i] : -1;
      }
      if (kEarlyRotate && bh != ready_bh) rotate_project<D, NW, QJ>(a, dv, b, h, s_q, s_pq, s_exp);
      const int nblk = (t1 - t0 + 15) >> 4;
#pragma unroll
      for (int r = 0; r < kStageRounds; ++r) {
        const int i = tid + r * NW * 64;
        if (i < nstage) s_blk[i] = (i < nblk && blk[r] >= 0 && (int64_t)blk[r] < pblocks) ? blk[r] : -1;
      }
      // every path through the masked stores above has its loads complete
      // here; otherwise the compiler keeps a load pending on the path that
      // skips a store and answers a later write of that register with a full
      // vmcnt wait, which would also wait for the first cache steps
      __builtin_amdgcn_s_waitcnt(kWaitVm0);
    }
    __syncthreads();
    if (cached) {
      // A operands (built while the first steps stream in): rows 0..GP-1 =
      // hi parts of head rows, GP..2GP-1 = lo parts.  A1[kt][m] slot e holds
      // coordinate 8 kt + 4 m + {0,1,0,1,2,3,2,3}[e] of the lane quarter,
      // matching the {hi pair, lo pair} B dwords; A3[kt] slot e holds
      // coordinate 8 kt + e (sign bits in order).  log2(e) sm_scale is folded
      // into q~, sqrt(pi/2) / d log2(e) sm_scale into p.
      auto setup = [&](bf16x8 (&A1r)[KT][2], bf16x8 (&A3r)[KT]) {
        if (bh == ready_bh) return;
        if (!kEarlyRotate) rotate_project<D, NW, QJ>(a, dv, b, h, s_q, s_pq, s_exp);
        const int arow = lane & 15, kq = lane >> 4;
        const int g = arow % GP;
        const bool is_lo = arow >= GP;
        const bool used = arow < 2 * GP && g < a.G;
        const float kappa = 1.2533141373155003f / (float)D;  // sqrt(pi/2) / d
        auto split = [&](float x) -> uint32_t {
          const float v = used ? x : 0.f;
          const uint32_t hb = f32_to_bf16_bits(v);
          return is_lo ? f32_to_bf16_bits(v - __uint_as_float(hb << 16)) : hb;
        };
        const float* xq = s_q + (used ? g : 0) * D;
        const float* yq = s_pq + (used ? g : 0) * D;
        float usum = 0.f;
#pragma unroll
        for (int kt = 0; kt < KT; ++kt) {
          const int j0 = kq * (D / 4) + 8 * kt;
          const f32x4 xa = *reinterpret_cast<const f32x4*>(xq + j0);
          const f32x4 xb = *reinterpret_cast<const f32x4*>(xq + j0 + 4);
          const f32x4 ya = *reinterpret_cast<const f32x4*>(yq + j0);
          const f32x4 yb = *reinterpret_cast<const f32x4*>(yq + j0 + 4);
          const float xs[8] = {xa[0], xa[1], xa[2], xa[3], xb[0], xb[1], xb[2], xb[3]};
          const float ys[8] = {ya[0], ya[1], ya[2], ya[3], yb[0], yb[1], yb[2], yb[3]};
          u32x4 w3;
          if constexpr (QJ) {
#pragma unroll
            for (int e = 0; e < 8; e += 2)
              w3[e / 2] = split(ys[e] * (kappa * a.logit_scale)) | (split(ys[e + 1] * (kappa * a.logit_scale)) << 16);
            A3r[kt] = __builtin_bit_cast(bf16x8, w3);
          }
          if constexpr (UN) {
            // slot 2j = coordinate j, slot 2j + 1 = coordinate j + 4 of the
            // slice (the code order of the arithmetic B operand), with the
            // codebook step folded in; usum collects the operand values
            const float ls = a.logit_scale * dv.uni_step;
            u32x4 w1;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
              const uint32_t lo = split(xs[j] * ls), hi = split(xs[j + 4] * ls);
              usum += __uint_as_float(lo << 16) + __uint_as_float(hi << 16);
              w1[j] = lo | (hi << 16);
            }
            A1r[kt][0] = __builtin_bit_cast(bf16x8, w1);
          } else if constexpr (KB == 8) {
            // slots 2e, 2e + 1 = coordinate 4m + e (against the {hi, lo} pair of c[idx])
#pragma unroll
            for (int m = 0; m < 2; ++m) {
              const float ls = a.logit_scale;
              u32x4 w;
#pragma unroll
              for (int e = 0; e < 4; ++e) {
                const uint32_t v = split(xs[4 * m + e] * ls);
                w[e] = v | (v << 16);
              }
              A1r[kt][m] = __builtin_bit_cast(bf16x8, w);
            }
          } else {
#pragma unroll
            for (int m = 0; m < 2; ++m) {
              const float ls = a.logit_scale;
              const uint32_t c01 = split(xs[4 * m] * ls) | (split(xs[4 * m + 1] * ls) << 16);
              const uint32_t c23 = split(xs[4 * m + 2] * ls) | (split(xs[4 * m + 3] * ls) << 16);
              A1r[kt][m] = __builtin_bit_cast(bf16x8, u32x4{c01, c01, c23, c23});
            }
          }
        }
        if constexpr (UN) {
          // Sum_j a_j (128 + idx_j) - (128 + (L-1)/2) Sum_j a_j
          //   = Sum_j a_j (idx_j - (L-1)/2) = Sum_j a_j (c[idx_j] - c0) / step + ...,
          // i.e. with c_k = (k - (L-1)/2) step the row's codebook term: the
          // offset is the accumulator's start value, per output row 4 (lane / 16) + r
          usum = lane_swap32_sum(lane_swap16_sum(usum));  // the row's operand sum (all 4 quarters)
          const float off = -(128.0f + 0.5f * (float)((1 << KB) - 1));
#pragma unroll
          for (int r = 0; r < 4; ++r) ucst[r] = off * __shfl(usum, 4 * kq + r);
        }
        // with lds_a, every wave stores the same operands to the shared copy
        // the steps read (no wave of the previous item reads it any more: the
        // item start is past the merge barrier)
#pragma unroll
        for (int kt = 0; kt < (lds_a<D, GP, KB, VB, QJ, UN>() ? KT : 0); ++kt) {
          s_A[(3 * kt) * 64 + lane] = __builtin_bit_cast(u32x4, A1r[kt][0]);
          if constexpr (!UN) s_A[(3 * kt + 1) * 64 + lane] = __builtin_bit_cast(u32x4, A1r[kt][1]);
          if constexpr (QJ) s_A[(3 * kt + 2) * 64 + lane] = __builtin_bit_cast(u32x4, A3r[kt]);
        }
        ready_bh = bh;
      };
      split_cached_chunk<D, GP, KB, VB, QJ, UN>(a, pr, h, t0, t1, s_blk, s_pair, s_sgn, s_p, s_main, s_stat, A1,
                                                A3, s_A, ucst, s_m, s_l, b, setup);
    } else if (!kDirect) {
      split_recent<D, GP, NW>(a, b, h, seq_recent(a, b), s_p, s_merge, s_m, s_l);
    }
    if (kDirect) {
      // the only split of this (sequence, KV head): acc / l is the output
      // (zero for a sequence with no tokens)
      for (int idx = tid; idx < a.G * D; idx += NW * 64) {
        const int g = idx / D;
        const float l = cached ? s_l[g] : 0.f;
        a.out[((int64_t)b * a.Hq + h * a.G) * D + idx] = l > 0.f ? s_merge[idx] / l : 0.f;
      }
    } else {
      // write the partial: (m, l, acc[D]) per query head of this KV head
      for (int idx = tid; idx < a.G * (D + 2); idx += NW * 64) {
        const int g = idx / (D + 2), k = idx % (D + 2);
        float v = k == 0 ? s_m[g] : (k == 1 ? s_l[g] : s_merge[g * D + (k - 2)]);
        a.part[(((int64_t)b * a.Hq + h * a.G + g) * a.splits_cap + c) * (D + 2) + k] = v;
      }
    }
    // Drain this item's stores here, where nothing else is in flight: the
    // compiler otherwise carries them into the next item and answers them
    // with full vmcnt waits after that item's first cache steps are
    // requested, which would also wait for those steps.
    __builtin_amdgcn_s_waitcnt(kWaitVm0);
    __syncthreads();
  };

  if (a.direct) {
    // one item per (sequence, KV head), contiguous ranges per workgroup: no
    // work list is needed
    store_table(tid);
    const int total = a.B * a.Hkv;
    const int i0 = (int)((int64_t)blockIdx.x * total / gridDim.x);
    const int i1 = (int)((int64_t)(blockIdx.x + 1) * total / gridDim.x);
    for (int item = i0; item < i1; ++item) {
      const int b = item / a.Hkv, h = item % a.Hkv;
      if (seq_preset_of(a, b) != pr) continue;  // uniform
      run_item(b, h, 0, seq_cached(a, b), std::true_type{});
    }
    return;
  }

  // work list: exclusive prefix over sequences of Hkv * splits(b) for the
  // sequences of this preset, in the (still unused) ring area
  int* s_scan = reinterpret_cast<int*>(s_main);
  {
    int carry = 0;
    for (int base = 0; base < a.B; base += NW * 64) {
      const int bb = base + tid;
      const int items = (bb < a.B && seq_preset_of(a, bb) == pr) ? a.Hkv * seq_splits(a, bb) : 0;
      int* sc = s_scan + base;
      if (bb < a.B) sc[tid] = items;
      if (base == 0) store_table(tid);
      __syncthreads();
      // Hillis-Steele inclusive scan of this block of 256 entries, in place
      for (int off = 1; off < NW * 64; off <<= 1) {
        const int v = (bb < a.B && tid >= off) ? sc[tid - off] : 0;
        __syncthreads();
        if (bb < a.B) sc[tid] += v;
        __syncthreads();
      }
      const int last = min(NW * 64, a.B - base) - 1;
      const int tot = sc[last];
      __syncthreads();
      if (bb < a.B) sc[tid] = carry + sc[tid] - items;  // exclusive
      carry += tot;
      __syncthreads();
    }
    if (tid == 0) s_scan[a.B] = carry;
    __syncthreads();
  }
  const int total = s_scan[a.B];
  const int i0 = (int)((int64_t)blockIdx.x * total / gridDim.x);
  const int i1 = (int)((int64_t)(blockIdx.x + 1) * total / gridDim.x);
  int b = 0, cur_base = 0;
  if (i0 < i1) {
    int lo = 0, hi = a.B - 1;  // largest b with s_scan[b] <= i0
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (s_scan[mid] <= i0) lo = mid; else hi = mid - 1;
    }
    b = lo;
    cur_base = s_scan[b];
  }
  __syncthreads();  // the ring area is free again

  for (int item = i0; item < i1; ++item) {
    // advance to the sequence holding this item (sequences of the other
    // preset, or with no splits, hold none)
    while (b < a.B && item - cur_base >= (seq_preset_of(a, b) == pr ? a.Hkv * seq_splits(a, b) : 0)) {
      cur_base += seq_preset_of(a, b) == pr ? a.Hkv * seq_splits(a, b) : 0;
      ++b;
    }
    if (b >= a.B) break;  // inconsistent with the scan: stop
    const int local = item - cur_base;
    const int nsp = seq_splits(a, b);
    run_item(b, local / nsp, local % nsp, seq_cached(a, b), std::false_type{});
  }
}

// ---------------------------------------------------------------------------
// combine: one workgroup per (sequence, query head).  Split weights
// 2^(m_s - M) are formed once in LDS (splits with l = 0 are empty and weigh 0),
// then each thread merges its channels.
// ---------------------------------------------------------------------------
constexpr int kCombineThreads = 128;
constexpr int kCombineMaxSplits = 1024;

#if TQ_DECODE_QJL
template <int D>
__global__ __launch_bounds__(kCombineThreads) void decode_combine_kernel(DArgs a) {
  __shared__ float s_w[kCombineMaxSplits];
  __shared__ float s_red[kCombineThreads];
  const int bh = blockIdx.x, tid = threadIdx.x;
  const int b = bh / a.Hq;
  const int ns = min(seq_splits(a, b), kCombineMaxSplits);
  const float* pp = a.part + (int64_t)bh * a.splits_cap * (D + 2);
  float mx = -INFINITY;
  for (int s = tid; s < ns; s += kCombineThreads) {
    const float l = pp[(int64_t)s * (D + 2) + 1];
    const float m = pp[(int64_t)s * (D + 2)];
    if (l > 0.f) mx = fmaxf(mx, m);
  }
  s_red[tid] = mx;
  __syncthreads();
  for (int off = kCombineThreads / 2; off > 0; off >>= 1) {
    if (tid < off) s_red[tid] = fmaxf(s_red[tid], s_red[tid + off]);
    __syncthreads();
  }
  const float M = s_red[0];
  __syncthreads();
  float lsum = 0.f;
  for (int s = tid; s < ns; s += kCombineThreads) {
    const float l = pp[(int64_t)s * (D + 2) + 1];
    const float w = l > 0.f ? __builtin_amdgcn_exp2f(pp[(int64_t)s * (D + 2)] - M) : 0.f;
    s_w[s] = w;
    lsum = __builtin_fmaf(w, l, lsum);
  }
  s_red[tid] = lsum;
  __syncthreads();
  for (int off = kCombineThreads / 2; off > 0; off >>= 1) {
    if (tid < off) s_red[tid] += s_red[tid + off];
    __syncthreads();
  }
  const float L = s_red[0];
  for (int c = tid; c < D; c += kCombineThreads) {
    float acc = 0.f;
#pragma unroll 4
    for (int s = 0; s < ns; ++s) acc = __builtin_fmaf(s_w[s], pp[(int64_t)s * (D + 2) + 2 + c], acc);
    a.out[(int64_t)bh * D + c] = L > 0.f ? acc / L : 0.f;
  }
}
#endif  // TQ_DECODE_QJL

// ---------------------------------------------------------------------------
// Launch configuration of one split kernel instantiation on one device,
// cached: its static LDS (the tables declared in the kernel), the dynamic LDS
// last granted with hipFuncSetAttribute, and workgroups per CU for the last
// dynamic size (from the occupancy calculator, so registers count as well as
// LDS).
struct SplitLaunchCache {
  std::mutex mu;
  struct Dev {
    bool init = false;
    int static_lds = 0, lds_limit = 0, cus = 0, granted = -1, occ_for = -1, per_cu = 1;
  } dev[16];
};

template <int D, int GP, int KB, int VB, bool QJ, bool UN = false>
static hipError_t launch_split(const DArgs& a, int pr, hipStream_t s, bool dry_run) {
  auto kern = decode_split_kernel<D, GP, KB, VB, QJ, UN>;
  using SL = SplitLds<D, GP, KB, VB, QJ, UN>;
  static SplitLaunchCache cache;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= 16) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(cache.mu);
  auto& c = cache.dev[dev];
  if (!c.init) {
    hipFuncAttributes attr{};
    if ((e = hipFuncGetAttributes(&attr, reinterpret_cast<const void*>(kern))) != hipSuccess) return e;
    c.static_lds = (int)attr.sharedSizeBytes;
    c.lds_limit = 160 * 1024;
    int v = 0;
    if (hipDeviceGetAttribute(&v, hipDeviceAttributeMaxSharedMemoryPerMultiprocessor, dev) == hipSuccess && v > 0)
      c.lds_limit = v;
    c.cus = 256;
    if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && v > 0) c.cus = v;
    c.init = true;
  }
  size_t lds = SL::total;
  const size_t recent_need = SL::kMainOffset + (size_t)(GP * a.W + GP * D) * 4;
  if (recent_need > lds) lds = recent_need;
  if ((int64_t)lds + c.static_lds > c.lds_limit) {
    set_error("decode: head_dim %d with %d query heads per KV head and recent_window %d needs %zu + %d bytes of LDS "
              "per workgroup (limit %d)", D, a.G, a.W, lds, c.static_lds, c.lds_limit);
    return hipErrorInvalidValue;
  }
  if (dry_run) return hipSuccess;
  if (c.granted != (int)lds) {
    e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern), hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    c.granted = (int)lds;
  }
  if (c.occ_for != (int)lds) {
    // persistent workgroups: as many as can be resident on the chip at once
    int nb = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, kern, SL::NW * 64, lds) != hipSuccess || nb < 1) nb = 1;
    c.per_cu = std::min(nb, 8);
    c.occ_for = (int)lds;
  }
  hipLaunchKernelGGL(kern, dim3(c.cus * c.per_cu), dim3(SL::NW * 64), lds, s, a, pr);
  return hipGetLastError();
}

template <int D, int GP, bool QJ>
static hipError_t dispatch_preset(const DArgs& a, int pr, int kb, int vb, hipStream_t s, bool dry) {
  if constexpr (!QJ)  // 8-bit keys: MSE-only presets
    if (kb == 8)
      return vb == 2 ? launch_split<D, GP, 8, 2, QJ>(a, pr, s, dry) : launch_split<D, GP, 8, 4, QJ>(a, pr, s, dry);
  // 4-bit equally spaced codebooks take the arithmetic score path
  if (kb == 4 && a.dev[pr].uni_step != 0.f)
    return vb == 2 ? launch_split<D, GP, 4, 2, QJ, true>(a, pr, s, dry) : launch_split<D, GP, 4, 4, QJ, true>(a, pr, s, dry);
  if (kb == 2) return vb == 2 ? launch_split<D, GP, 2, 2, QJ>(a, pr, s, dry) : launch_split<D, GP, 2, 4, QJ>(a, pr, s, dry);
  if (kb == 3) return vb == 2 ? launch_split<D, GP, 3, 2, QJ>(a, pr, s, dry) : launch_split<D, GP, 3, 4, QJ>(a, pr, s, dry);
  return vb == 2 ? launch_split<D, GP, 4, 2, QJ>(a, pr, s, dry) : launch_split<D, GP, 4, 4, QJ>(a, pr, s, dry);
}

// The split launches of one key kind.  This source is compiled twice, with
// TQ_DECODE_QJL = 1 (keys with the QJL sketch; this object also holds the
// combine kernel and the entry point) and = 0 (MSE-only keys), so that no
// kernel is instantiated in both objects.
// dry = true only checks that the launch fits (LDS) and enqueues nothing.
hipError_t launch_split_qjl(const DArgs& a, int pr, int d, int G, int kb, int vb, hipStream_t s, bool dry);
hipError_t launch_split_mse(const DArgs& a, int pr, int d, int G, int kb, int vb, hipStream_t s, bool dry);

#if TQ_DECODE_QJL
hipError_t launch_split_qjl(const DArgs& a, int pr, int d, int G, int kb, int vb, hipStream_t s, bool dry) {
  if (d == 128) return G <= 4 ? dispatch_preset<128, 4, true>(a, pr, kb, vb, s, dry) : dispatch_preset<128, 8, true>(a, pr, kb, vb, s, dry);
  return G <= 4 ? dispatch_preset<256, 4, true>(a, pr, kb, vb, s, dry) : dispatch_preset<256, 8, true>(a, pr, kb, vb, s, dry);
}
#else
hipError_t launch_split_mse(const DArgs& a, int pr, int d, int G, int kb, int vb, hipStream_t s, bool dry) {
  if (d == 128) return G <= 4 ? dispatch_preset<128, 4, false>(a, pr, kb, vb, s, dry) : dispatch_preset<128, 8, false>(a, pr, kb, vb, s, dry);
  return G <= 4 ? dispatch_preset<256, 4, false>(a, pr, kb, vb, s, dry) : dispatch_preset<256, 8, false>(a, pr, kb, vb, s, dry);
}
#endif

#if TQ_DECODE_QJL
// dry = true: only check that every split launch fits (no work enqueued).
template <int D>
static hipError_t launch_all(const DArgs& a0, const tq_decode_args* args, hipStream_t s, bool dry) {
  hipError_t e = hipSuccess;
  // with no recent window and max_seq_len <= chunk every sequence has at most
  // one split (cached lengths are clamped to max_seq_len): the split kernel
  // then writes the output itself and the combine pass is skipped
  DArgs a = a0;
  a.direct = (args->recent_k == nullptr && args->max_seq_len <= args->chunk_tokens) ? 1 : 0;
  for (int pr = 0; pr < args->num_presets; ++pr) {
    const tq_ctx* c = args->ctx[pr];
    e = c->qjl ? launch_split_qjl(a, pr, D, a.G, c->kb, c->vb, s, dry)
               : launch_split_mse(a, pr, D, a.G, c->kb, c->vb, s, dry);
    if (e != hipSuccess) return e;
  }
  if (a.direct || dry) return hipSuccess;
  hipLaunchKernelGGL(decode_combine_kernel<D>, dim3(a.B * a.Hq), dim3(kCombineThreads), 0, s, a);
  return hipGetLastError();
}

static DArgs make_dargs(const tq_decode_args* args, const DecodePlan& plan) {
  DArgs a{};
  a.q = args->q;
  a.q_bf16 = args->q_dtype == TQ_DTYPE_BF16;
  a.B = args->batch;
  a.Hq = args->num_q_heads;
  a.Hkv = args->num_kv_heads;
  a.G = a.Hq / a.Hkv;
  for (int i = 0; i < 2; ++i) {
    const tq_ctx* c = args->ctx[i < args->num_presets ? i : 0];
    a.pool[i] = reinterpret_cast<const uint8_t*>(args->pool[i < args->num_presets ? i : 0]);
    a.pool_blocks[i] = args->pool_blocks[i < args->num_presets ? i : 0];
    a.rec[i] = c->lay.bytes;
    a.lay[i] = c->lay;
    a.dev[i] = c->dev;
  }
  a.seq_preset = args->num_presets == 2 ? args->seq_preset : nullptr;
  a.bt = args->block_tables;
  a.max_blocks = args->max_blocks_per_seq;
  a.seq_lens = args->seq_lens;
  a.max_seq_len = args->max_seq_len;
  a.rk = args->recent_k;
  a.rv = args->recent_v;
  a.rlens = args->recent_lens;
  a.W = args->recent_k ? args->recent_window : 0;
  a.sm_scale = args->sm_scale > 0.f ? args->sm_scale : 1.0f / std::sqrt((float)plan.d);
  a.logit_scale = a.sm_scale * 1.4426950408889634f;
  a.inv_logit_scale = 1.f / a.logit_scale;
  a.chunk = args->chunk_tokens;
  a.splits_cap = plan.num_splits_max;
  char* ws = reinterpret_cast<char*>(args->workspace);
  a.part = reinterpret_cast<float*>(ws + plan.off_part);
  a.out = args->out;
  a.scores = args->scores_out;
  a.scores_stride = args->scores_stride;
  return a;
}

// Split partials of tq_decode_attention_noalloc: a file-scope device array
// (each GPU holds its own copy at its own address until the process ends).
// Host code never uses the array's name as an address: the per-device
// address comes from hipGetSymbolAddress, with that device current.
static __device__ __align__(256) unsigned char scratch[TQ_NOALLOC_SCRATCH_BYTES];

hipError_t noalloc_scratch(void** out) {
  static std::mutex mu;
  static void* addr[16] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= 16) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    addr[dev] = p;
  }
  *out = addr[dev];
  return hipSuccess;
}

hipError_t check_decode_launch(const tq_decode_args* args, const DecodePlan& plan) {
  const DArgs a = make_dargs(args, plan);
  return plan.d == 128 ? launch_all<128>(a, args, nullptr, true) : launch_all<256>(a, args, nullptr, true);
}

hipError_t launch_decode(const tq_decode_args* args, const DecodePlan& plan, hipStream_t stream) {
  const DArgs a = make_dargs(args, plan);
  return plan.d == 128 ? launch_all<128>(a, args, stream, false) : launch_all<256>(a, args, stream, false);
}
#endif  // TQ_DECODE_QJL

}  // namespace tq
