// Fused quantise + pack + paged store for large batches of bf16 keys and
// values at head_dim 128 (Roadmap §3.1: the rotation fused with the quantiser
// in the store launch; Hub, technical principle steps 1-5), with both dense
// products of the key path on the matrix cores.
//
// A wave owns a tile of 16 consecutive tokens of one KV head.  In the MFMA
// layout lane l plays row n = l % 16 (a token) and group g = l / 16:
//   rotation  y = H D1 k on v_mfma_f32_16x16x32_bf16, computed transposed:
//             C[j][n] = sum_k H[j][k] (D1 k_n)[k].  The B operand is the bf16
//             key itself (lane (n, g) loads coordinates 32 kt + 8 g .. + 7 of
//             its row, D1 applied as a sign-bit xor), products are exact and
//             the sums fp32.  The A operand is the Sylvester Hadamard matrix:
//             H[16 nt + m][32 kt + k] = (-1)^popcount(nt & (2 kt + k / 16))
//             (-1)^popcount(m & (k % 16)), so every A tile is one of four
//             per-lane sign patterns held in registers.  Lane (n, g) receives
//             coordinates 16 nt + 4 g + r (nt < 8, r < 4) of row n.
//   quantise  as the other store kernels: norm, Lloyd-Max index of the
//             D2-free coordinate from its magnitude, residual, gamma.
//   QJL       z = S r on v_mfma_f32_16x16x32_f16 with the residual as the B
//             operand straight from the registers the rotation left it in:
//             k-slice kt, element e of lane (n, g) is coordinate
//             32 kt + 16 (e / 4) + 4 g + e % 4, and the context's S tiles are
//             laid out with the same permutation of the k index (D2 folded in,
//             fp16 hi / lo of 16 S, three products per slice).  Lane (n, g)
//             gets z_i for i = 16 nt + 4 g + r and packs its sign bits.
//   pack      code and sign-bit fields are placed at their stream offsets in
//             the lane and or-ed over the four lanes of a row (permlane swaps).
// The key rows of a wave's next tile are copied into its LDS buffer while the
// current tile runs (global_load_lds), so tiles start without a key round trip.
// Values are quantised in the row-part layout (lane: row l / 4, 32-channel
// group l % 4), one group per lane.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <mutex>

#include "tq_common.hip.h"
#include "tq_internal.h"

namespace tq {
namespace {

typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

constexpr int MD = 128, MKT = 4, MNT = 8;
// waves per workgroup: with the QJL tiles (64 KB of LDS) one workgroup fills a
// CU at three waves per SIMD; MSE-only keys need no tiles and run 8-wave
// workgroups, several per CU
template <bool QJ>
constexpr int mwaves() {
  return QJ ? 12 : 8;
}

struct QMArgs {
  const uint16_t* k;
  const uint16_t* v;
  int64_t num_tokens;
  int32_t hkv;
  const int32_t* slot_mapping;
  int64_t slots_total;
  uint8_t* pool;
  int64_t rec;
  Layout lay;
  DevTables dev;
  int64_t num_tiles;
};

// sum over the four lanes l, l ^ 16, l ^ 32, l ^ 48 (the lanes of one row)
__device__ __forceinline__ float row_sum4(float x) {
  auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}
// Two or-reductions with one lane exchange.  Across the wave halves: lanes
// 0..31 get a[l] | a[l + 32], lanes 32..63 get b[l - 32] | b[l].
__device__ __forceinline__ uint32_t or_halves(uint32_t a, uint32_t b) {
  auto s = __builtin_amdgcn_permlane32_swap(a, b, false, false);
  return s[0] | s[1];
}
// Across 16-lane row pairs: row 0 gets a.r0 | a.r1, row 1 b.r0 | b.r1, row 2
// a.r2 | a.r3, row 3 b.r2 | b.r3.
__device__ __forceinline__ uint32_t or_row_pairs(uint32_t a, uint32_t b) {
  auto s = __builtin_amdgcn_permlane16_swap(a, b, false, false);
  return s[0] | s[1];
}
constexpr int parity(int x) { return __builtin_popcount(x) & 1; }
// The code-stream dword that lane group g stores as its i-th (see the packing
// of each key width below).
template <int KB>
__device__ __forceinline__ int stream_dword(int g, int i) {
  constexpr int CPL = KB * 128 / 32 / 4;
  if constexpr (KB == 4) return 2 * (CPL * (g & 1) + i) + (g >> 1);
  if constexpr (KB == 8) return 4 * i + g;
  return CPL * g + i;
}
// LDS: the QJL tiles (64 KB), the upper centroids (and, for 8-bit codes, the
// upper thresholds), the row's D2 code patterns
template <int KB, bool QJ>
constexpr int m_lds_m2() {
  return (QJ ? 65536 : 0) + (KB <= 4 ? 64 : 1024);
}
// then each wave's buffer for the key rows of its next tile (16 rows x d bf16)
template <int KB, bool QJ>
constexpr int m_lds_kbuf() {
  return (m_lds_m2<KB, QJ>() + KB * MD / 8 + 15) / 16 * 16;
}
constexpr int kKeyTileBytes = 16 * MD * 2;
template <int KB, bool QJ>
constexpr int m_lds_bytes() {
  return m_lds_kbuf<KB, QJ>() + mwaves<QJ>() * kKeyTileBytes;
}
// Direct global -> LDS copy of 16 bytes per lane (lane l's bytes land at LDS
// byte address m0 + 16 l), as inline assembly so that the compiler does not
// fence later LDS reads on it; completion is awaited with s_waitcnt vmcnt.
__device__ __forceinline__ void key_dma16(uint32_t lds_byte_addr, uint64_t sbase, uint32_t voff) {
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)sbase);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(sbase >> 32));
  asm volatile(
      "s_mov_b32 m0, %0\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %2, %1"
      :
      : "s"((uint32_t)__builtin_amdgcn_readfirstlane((int)lds_byte_addr)), "s"(((uint64_t)hi << 32) | (uint64_t)lo),
        "v"(voff)
      : "memory");
}

template <int KB, int VB, bool QJ>
__global__ __launch_bounds__(mwaves<QJ>() * 64) void quantize_mfma_kernel(QMArgs a) {
  constexpr int MW = mwaves<QJ>();
  constexpr int L = 1 << KB, H = L / 2;
  extern __shared__ __attribute__((aligned(16))) unsigned char lds[];
  const u32x4* s_st = reinterpret_cast<const u32x4*>(lds);          // [nt][kt][hi, lo][64] (QJL)
  float* s_c = reinterpret_cast<float*>(lds + (QJ ? 65536 : 0));     // c[H .. L-1]
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int n = lane & 15, g = lane >> 4;

  if constexpr (QJ) {
    const u32x4* src = reinterpret_cast<const u32x4*>(a.dev.s_tiles_perm_d2);
    for (int i = tid; i < 4096; i += MW * 64) const_cast<u32x4*>(s_st)[i] = src[i];
  }
  // upper centroids in LDS; upper thresholds in registers (8-bit codes: in
  // LDS after the centroids, for a binary search).  The key path works on
  // coordinates scaled by the power of two R = 2^kRScaleLog2 that the QJL
  // operands need, so centroids and thresholds are scaled by R here (exact:
  // every decision and rounding is the same as unscaled, times R).
  const float rscale = (float)(1 << kRScaleLog2);
  float* s_tU = s_c + H;
  if (tid < H) s_c[tid] = a.dev.centroids[H + tid] * rscale;
  float tU[KB <= 4 ? H - 1 : 1];
  if constexpr (KB <= 4) {
#pragma unroll
    for (int i = 0; i < H - 1; ++i) tU[i] = a.dev.thresholds[H + i] * rscale;
  } else {
    tU[0] = 0.f;
    if (tid < H - 1) s_tU[tid] = a.dev.thresholds[H + tid] * rscale;
  }
  // D1 as bf16 sign-bit masks of the key operand: element e of slice kt is
  // coordinate 32 kt + 8 g + e
  u32x4 d1m[MKT];
#pragma unroll
  for (int kt = 0; kt < MKT; ++kt)
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const int c0 = 32 * kt + 8 * g + 2 * w;
      d1m[kt][w] = (a.dev.signs1[c0] < 0.f ? 0x8000u : 0u) | (a.dev.signs1[c0 + 1] < 0.f ? 0x80000000u : 0u);
    }
  // Hadamard A patterns: element e of lane (m = n, g) is (-1)^popcount(m & (8 (g & 1) + e)),
  // times the tile sign of the lane's half (g >> 1): hv[s0][s1] takes sign s0
  // on lanes g < 2 and s1 on lanes g >= 2
  u32x4 hv[2][2];
  {
    u32x4 pos;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      uint32_t d = 0;
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int e = 2 * w + u;
        const uint32_t neg = (uint32_t)(__builtin_popcount(n & (8 * (g & 1) + e)) & 1);
        d |= (neg ? 0xBF80u : 0x3F80u) << (16 * u);
      }
      pos[w] = d;
    }
#pragma unroll
    for (int s0 = 0; s0 < 2; ++s0)
#pragma unroll
      for (int s1 = 0; s1 < 2; ++s1) {
        const uint32_t flip = ((g >> 1) ? s1 : s0) ? 0x80008000u : 0u;
#pragma unroll
        for (int w = 0; w < 4; ++w) hv[s0][s1][w] = pos[w] ^ flip;
      }
  }
  // D2 as code-word xor patterns of the row's code stream (index ^ (L - 1)
  // where D2 = -1; the kernel works on D2-free coordinates), or-ed together in
  // LDS by one thread per coordinate
  constexpr int CWD = KB * MD / 32;   // code dwords per row
  constexpr int CPL = CWD / 4;        // code dwords stored per lane
  uint32_t* s_m2 = reinterpret_cast<uint32_t*>(lds + m_lds_m2<KB, QJ>());
  if (tid < CWD) s_m2[tid] = 0;
  __syncthreads();
  if (tid < MD && a.dev.signs2[tid] < 0.f) {
    const int bp = tid * KB;
    atomicOr(&s_m2[bp / 32], (uint32_t)(L - 1) << (bp % 32));
    if ((bp % 32) + KB > 32) atomicOr(&s_m2[bp / 32 + 1], (uint32_t)(L - 1) >> (32 - bp % 32));
  }
  __syncthreads();
  uint32_t m2c[CPL];  // the patterns of the stream dwords this lane stores
#pragma unroll
  for (int i = 0; i < CPL; ++i) m2c[i] = s_m2[stream_dword<KB>(g, i)];

  const float inv_sqrt_d = 1.0f / __builtin_sqrtf((float)MD);
  // A tile is 16 consecutive tokens of one KV head (so that, when their slots
  // fill a paged block in order, every region of the block's record is
  // written by this wave in contiguous runs): tile = token block * hkv + head.
  // The wave's tiles advance by a fixed stride, so the (token block, head)
  // pair advances by the stride's quotient and remainder.
  const int64_t tstride = (int64_t)gridDim.x * MW;
  const int64_t tile0 = (int64_t)blockIdx.x * MW + __builtin_amdgcn_readfirstlane(wave);
  const int64_t blk_step = tstride / a.hkv;
  const int head_step = (int)(tstride % a.hkv);
  int64_t tblk = tile0 / a.hkv;
  int hh = (int)(tile0 % a.hkv);
  // The key rows of a wave's next tile are copied to its LDS buffer while the
  // current tile is processed (lane (n, g) copies row n's coordinates
  // 32 kt + 8 g .. + 7 for kt < 4; rows past the batch copy row t0 instead).
  unsigned char* kbuf = lds + m_lds_kbuf<KB, QJ>() + __builtin_amdgcn_readfirstlane(wave) * kKeyTileBytes;
  const uint32_t kbuf_addr = (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)kbuf;
  auto fetch_keys = [&](int64_t tb, int hd) {
    const int64_t row0 = tb * 16;
    const int64_t r = row0 + n < a.num_tokens ? n : 0;
    const uint64_t sbase = (uint64_t)(uintptr_t)(a.k + (row0 * a.hkv + hd) * MD);
    const uint32_t voff = (uint32_t)((r * a.hkv * MD + 8 * g) * 2);
#pragma unroll
    for (int kt = 0; kt < MKT; ++kt) key_dma16(kbuf_addr + kt * 1024, sbase, voff + kt * 64);
  };
  if (tile0 < a.num_tiles) fetch_keys(tblk, hh);
  for (int64_t tile = tile0; tile < a.num_tiles;
       tile += tstride, tblk += blk_step + (hh + head_step >= a.hkv ? 1 : 0),
               hh = hh + head_step >= a.hkv ? hh + head_step - a.hkv : hh + head_step) {
    const int64_t t0 = tblk * 16;
    // ---------------------------------------------------------------- key
    const int64_t tk = t0 + n;
    const bool valid = tk < a.num_tokens;
    // value rows: lane l holds channels 32 (l % 4) .. + 31 of row l / 4
    const int vrow = lane >> 2, vpart = lane & 3;
    const int64_t tv = t0 + vrow;
    const bool vvalid = tv < a.num_tokens;
    // Every global read of the tile is issued before its first store (the
    // compiler cannot move a read above a store it cannot prove disjoint):
    // the key rows and both rows' slots here, the value rows right after the
    // rotation, so the tile waits for one memory round trip instead of four.
    const int32_t slot = valid ? a.slot_mapping[tk] : -1;
    const int32_t vslot = vvalid ? a.slot_mapping[tv] : -1;
    bf16x8 kbv[MKT];
    {
      // this tile's key rows, then the copy of the next tile's into the same
      // buffer once they are read.  The copy issued during the previous tile
      // completed at that tile's wait before its value stage (below), so
      // only the first tile waits here, and no tile waits at its start for
      // the previous tile's record stores.
      if (tile == tile0) asm volatile("s_waitcnt vmcnt(0)" : : : "memory");
      u32x4 kw[MKT];
#pragma unroll
      for (int kt = 0; kt < MKT; ++kt) kw[kt] = *reinterpret_cast<const u32x4*>(kbuf + kt * 1024 + lane * 16);
      asm volatile("s_waitcnt lgkmcnt(0)" : : : "memory");
      if (tile + tstride < a.num_tiles) {  // uniform
        const int nh = hh + head_step;
        fetch_keys(tblk + blk_step + (nh >= a.hkv ? 1 : 0), nh >= a.hkv ? nh - a.hkv : nh);
      }
#pragma unroll
      for (int kt = 0; kt < MKT; ++kt) {
        u32x4 w = valid ? kw[kt] : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
        for (int i = 0; i < 4; ++i) w[i] ^= d1m[kt][i];
        kbv[kt] = __builtin_bit_cast(bf16x8, w);
      }
    }
    f32x4 y[MNT];
#pragma unroll
    for (int nt = 0; nt < MNT; ++nt) {
      y[nt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kt = 0; kt < MKT; ++kt) {
        const u32x4 hp = hv[parity(nt & (2 * kt))][parity(nt & (2 * kt + 1))];
        y[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, hp), kbv[kt], y[nt], 0, 0, 0);
      }
    }
    u32x4 vraw[4];
    {
      const u32x4* pv = reinterpret_cast<const u32x4*>(a.v + (vvalid ? tv * a.hkv + hh : 0) * MD + 32 * vpart);
#pragma unroll
      for (int i = 0; i < 4; ++i) vraw[i] = vvalid ? __builtin_nontemporal_load(pv + i) : u32x4{0u, 0u, 0u, 0u};
    }
    // norm: sum of squares of the rotated row (H H^T = d I) over the row's lanes
    float ss = 0.f;
#pragma unroll
    for (int nt = 0; nt < MNT; ++nt)
#pragma unroll
      for (int r = 0; r < 4; ++r) ss = __builtin_fmaf(y[nt][r], y[nt][r], ss);
    ss = row_sum4(ss);
    const float nrm = __builtin_sqrtf(ss * (1.0f / MD));
    const bool zero = !(nrm > 0.f);
    const float inv = zero ? 0.f : (inv_sqrt_d / nrm) * rscale;  // R / (sqrt(d) n)
    // Lloyd-Max index of the D2-free coordinate from its magnitude, and the residual
    uint32_t field[MNT];
    float r2 = 0.f;
#pragma unroll
    for (int nt = 0; nt < MNT; ++nt) {
      field[nt] = 0;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float u = y[nt][r] * inv;
        const float m = fabsf(u);
        uint32_t cnt = 0;
        if constexpr (KB <= 4) {
          // #{upper thresholds < m} by binary search over the sorted
          // thresholds in registers (each level picks its threshold with
          // selects on the bits found so far)
          if constexpr (H == 2) {
            cnt = m > tU[0] ? 1u : 0u;
          } else if constexpr (H == 4) {
            const bool b1 = m > tU[1];
            const float t = b1 ? tU[2] : tU[0];
            cnt = (b1 ? 2u : 0u) + (m > t ? 1u : 0u);
          } else {
            const bool b2 = m > tU[3];
            const float t1 = b2 ? tU[5] : tU[1];
            const bool b1 = m > t1;
            const float t0 = b2 ? (b1 ? tU[6] : tU[4]) : (b1 ? tU[2] : tU[0]);
            cnt = (b2 ? 4u : 0u) + (b1 ? 2u : 0u) + (m > t0 ? 1u : 0u);
          }
        } else {
          // #{upper thresholds < m}: seven halving steps over the 127 in LDS
#pragma unroll
          for (int st = H / 2; st >= 1; st >>= 1) cnt += m > s_tU[cnt + st - 1] ? (uint32_t)st : 0u;
        }
        const float dd = m - s_c[cnt];
        const bool pos = u > 0.f;
        const uint32_t code = cnt ^ (pos ? (uint32_t)H : (uint32_t)H - 1u);
        float res = pos ? dd : -dd;
        r2 = __builtin_fmaf(res, res, r2);
        y[nt][r] = res;
        field[nt] |= code << (KB * r);
      }
    }
    // a zero key stores zero codes, sign bits and gamma (selected per row
    // below, not per coordinate)
    // (r2 holds R^2 |r|^2: the root scales exactly by R)
    const float gamma = zero ? 0.f : __builtin_sqrtf(row_sum4(r2)) * (1.0f / rscale);

    // ---- QJL sign bits of S r (MSE-only keys skip the sketch)
    uint32_t qw = 0;  // the sign dword this lane stores (dword g of the row's d / 8 bytes)
    if constexpr (QJ) {
      // fp16 hi / lo parts of R r, two elements per packed conversion
      f16x8 rbh[MKT], rbl[MKT];
#pragma unroll
      for (int kt = 0; kt < MKT; ++kt)
#pragma unroll
        for (int e = 0; e < 8; e += 2) {
          const f32x2 x = {y[2 * kt + (e >> 2)][e & 3], y[2 * kt + (e >> 2)][(e & 3) + 1]};
          const f16x2 xh = __builtin_convertvector(x, f16x2);
          const f16x2 xl = __builtin_convertvector(x - __builtin_convertvector(xh, f32x2), f16x2);
          rbh[kt][e] = xh[0];
          rbh[kt][e + 1] = xh[1];
          rbl[kt][e] = xl[0];
          rbl[kt][e + 1] = xl[1];
        }
      // one column tile of z at a time (the S tiles come from LDS per tile);
      // bit i = 16 nt + 4 g + r of the row's stream is bit 16 (nt % 2) + 4 g + r
      // of dword nt / 2, which lane g = nt / 2 keeps
      // dword p (of the row's four sign dwords) gets bits 16 (nt % 2) + 4 g + r
      // of column tiles nt = 2 p, 2 p + 1 from every lane group g; the four
      // partial dwords rotate through d0..d3 and one reduce-scatter over the
      // row's lanes leaves dword g in lane group g
      uint32_t d0 = 0, d1 = 0, d2 = 0, d3 = 0;
#pragma unroll 1
      for (int p = 0; p < MNT / 2; ++p) {
        uint32_t dw = 0;
#pragma unroll
        for (int hn = 0; hn < 2; ++hn) {
          const int nt = 2 * p + hn;
          f32x4 z = {0.f, 0.f, 0.f, 0.f};
          const u32x4* tp = s_st + (nt * MKT * 2) * 64 + lane;
#pragma unroll
          for (int kt = 0; kt < MKT; ++kt) {
            const f16x8 ah = __builtin_bit_cast(f16x8, tp[(2 * kt) * 64]);
            const f16x8 al = __builtin_bit_cast(f16x8, tp[(2 * kt + 1) * 64]);
            z = __builtin_amdgcn_mfma_f32_16x16x32_f16(ah, rbh[kt], z, 0, 0, 0);
            z = __builtin_amdgcn_mfma_f32_16x16x32_f16(ah, rbl[kt], z, 0, 0, 0);
            z = __builtin_amdgcn_mfma_f32_16x16x32_f16(al, rbh[kt], z, 0, 0, 0);
          }
          uint32_t nib = 0;
#pragma unroll
          for (int r = 0; r < 4; ++r) nib |= (z[r] >= 0.f ? 1u : 0u) << r;
          dw |= nib << (16 * hn + 4 * g);
        }
        d0 = d1;
        d1 = d2;
        d2 = d3;
        d3 = dw;
      }
      qw = or_row_pairs(or_halves(d0, d2), or_halves(d1, d3));
      qw = zero ? 0u : qw;
    }

    // ---- code stream of the row: field nt (4 codes) at bit KB (16 nt + 4 g).
    // Each lane places its fields in the stream dwords they fall into; the
    // or over the row's four lanes is a reduce-scatter with lane exchanges,
    // leaving in lane group g exactly the dwords it stores.
    uint32_t cst[CPL];
    if constexpr (KB == 2) {
      // 8-bit fields: dword nt, byte g; lane g stores dwords 2 g, 2 g + 1
      uint32_t h[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) h[k] = or_halves(field[k] << (8 * g), field[k + 4] << (8 * g));
#pragma unroll
      for (int i = 0; i < CPL; ++i) cst[i] = or_row_pairs(h[i], h[i + 2]);
    } else if constexpr (KB == 3) {
      // pairs of 12-bit fields in three dwords 3 p .. 3 p + 2: F_2p at bit 12 g,
      // F_2p+1 at bit 48 + 12 g; lane g stores dwords 3 g .. 3 g + 2
      uint32_t c[12];
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        const uint64_t x = (uint64_t)field[2 * p] | ((uint64_t)field[2 * p + 1] << 48);
        const uint64_t lo = x << (12 * g);
        c[3 * p] = (uint32_t)lo;
        c[3 * p + 1] = (uint32_t)(lo >> 32);
        c[3 * p + 2] = (uint32_t)(((uint64_t)field[2 * p + 1] << (12 * g + 16)) >> 32);
      }
      uint32_t h[6];
#pragma unroll
      for (int k = 0; k < 6; ++k) h[k] = or_halves(c[k], c[k + 6]);
#pragma unroll
      for (int i = 0; i < CPL; ++i) cst[i] = or_row_pairs(h[i], h[i + 3]);
    } else if constexpr (KB == 8) {
      // 32-bit fields: the lane's four codes of column tile nt are bytes
      // 16 nt + 4 g .. + 3 of the stream, i.e. dword 4 nt + g, whole
#pragma unroll
      for (int i = 0; i < CPL; ++i) cst[i] = field[i];
    } else {
      // 16-bit fields: dword 2 nt + (g >> 1), half g & 1 (an or over the lane
      // pair g, g ^ 1); lane g stores dwords 2 (4 (g & 1) + i) + (g >> 1), i < 4
#pragma unroll
      for (int i = 0; i < CPL; ++i) cst[i] = or_row_pairs(field[i] << (16 * (g & 1)), field[4 + i] << (16 * (g & 1)));
    }

    // -------------------------------------------------------------- value
    // the value rows, the slots and the next tile's key copy were all issued
    // before any store of this tile: this waits for loads only
    asm volatile("s_waitcnt vmcnt(0)" : : : "memory");
    // row-part layout: lane l holds channels 32 (l % 4) .. + 31 of row l / 4
    {
      const int part = vpart;
      float x[32];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          x[8 * i + 2 * j] = __uint_as_float(vraw[i][j] << 16);
          x[8 * i + 2 * j + 1] = __uint_as_float(vraw[i][j] & 0xFFFF0000u);
        }
      }
      constexpr float LV = (float)((1 << VB) - 1);
      float mn = x[0], mx = x[0];
#pragma unroll
      for (int e = 1; e < 32; ++e) {
        mn = fminf(mn, x[e]);
        mx = fmaxf(mx, x[e]);
      }
      const uint16_t s16 = f32_to_f16_bits((mx - mn) / LV);
      const uint16_t z16 = f32_to_f16_bits(mn);
      const float sc = f16_bits_to_f32(s16), zz = f16_bits_to_f32(z16);
      // q = rint((v - z) / s) with the IEEE quotient, from the product with
      // the rounded reciprocal and one correction by the exact residual
      // (Markstein's theorem: the corrected quotient is the correctly rounded
      // one; checked for every fp16 scale around every half-integer).  A
      // constant group (s = 0) codes 0: with rs = 0 every quotient is 0.
      const float rs = sc != 0.f ? 1.0f / sc : 0.f;
      uint32_t vw[VB];
#pragma unroll
      for (int i = 0; i < VB; ++i) vw[i] = 0;
#pragma unroll
      for (int e = 0; e < 32; ++e) {
        const float dv = x[e] - zz;
        const float q0 = dv * rs;
        const float t = __builtin_fmaf(__builtin_fmaf(-q0, sc, dv), rs, q0);
        const float q = fminf(fmaxf(__builtin_rintf(t), 0.f), LV);
        vw[(e * VB) / 32] |= (uint32_t)q << ((e * VB) % 32);
      }
      // ---- store the key record (after the value arithmetic: a wait for the
      // value rows issued after these stores would also wait for the stores)
      if (valid && slot >= 0 && (int64_t)slot < a.slots_total) {
        uint8_t* base = a.pool + ((int64_t)(slot >> 4) * a.hkv + hh) * a.rec;
        const int s = slot & 15;
        uint8_t* kc = base + a.lay.kcodes + s * (KB * MD / 8);
#pragma unroll
        for (int i = 0; i < CPL; ++i) {
          const int wd = stream_dword<KB>(g, i);
          *reinterpret_cast<uint32_t*>(kc + 4 * wd) = zero ? 0u : (cst[i] ^ m2c[i]);
        }
        if constexpr (QJ) {
          *reinterpret_cast<uint32_t*>(base + a.lay.kqjl + s * (MD / 8) + 4 * g) = qw;
          if (g == 0)
            *reinterpret_cast<uint32_t*>(base + a.lay.kmeta + s * 4) =
                (uint32_t)f32_to_f16_bits(zero ? 0.f : nrm) | ((uint32_t)f32_to_f16_bits(gamma) << 16);
        } else if (g == 0) {
          *reinterpret_cast<uint16_t*>(base + a.lay.kmeta + s * 2) = f32_to_f16_bits(zero ? 0.f : nrm);
        }
      }
      if (vvalid && vslot >= 0 && (int64_t)vslot < a.slots_total) {
        uint8_t* base = a.pool + ((int64_t)(vslot >> 4) * a.hkv + hh) * a.rec;
        const int s = vslot & 15;
#pragma unroll
        for (int i = 0; i < VB; ++i)
          *reinterpret_cast<uint32_t*>(base + a.lay.vcodes + ((part * VB + i) * 16 + s) * 4) = vw[i];
        *reinterpret_cast<uint32_t*>(base + a.lay.vmeta + (part * 16 + s) * 4) = (uint32_t)s16 | ((uint32_t)z16 << 16);
      }
    }
  }
}

template <int KB, int VB, bool QJ>
hipError_t launch_m(const QMArgs& a, hipStream_t stream) {
  constexpr int MW = mwaves<QJ>();
  auto kern = quantize_mfma_kernel<KB, VB, QJ>;
  const int lds = m_lds_bytes<KB, QJ>();
  struct Cache {
    std::mutex mu;
    bool init[16] = {};
    int grid[16] = {};
  };
  static Cache cache;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= 16) return hipErrorInvalidDevice;
  int slots;
  {
    std::lock_guard<std::mutex> lock(cache.mu);
    if (!cache.init[dev]) {
      e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern), hipFuncAttributeMaxDynamicSharedMemorySize, lds);
      if (e != hipSuccess) return e;
      int cus = 256, per = 1;
      (void)hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
      if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per, kern, MW * 64, lds) != hipSuccess || per < 1) per = 1;
      cache.grid[dev] = cus * per;
      cache.init[dev] = true;
    }
    slots = cache.grid[dev];
  }
  // persistent workgroups: as many as are resident at once, or fewer
  const int64_t want = (a.num_tiles + MW - 1) / MW;
  const int grid = (int)std::min<int64_t>(want, (int64_t)slots);
  if (grid <= 0) return hipSuccess;
  hipLaunchKernelGGL(kern, dim3(grid), dim3(MW * 64), lds, stream, a);
  return hipGetLastError();
}

template <bool QJ>
hipError_t dispatch_m(const QMArgs& a, int kb, int vb, hipStream_t s) {
  if constexpr (!QJ)  // 8-bit keys: MSE-only presets
    if (kb == 8) return vb == 2 ? launch_m<8, 2, QJ>(a, s) : launch_m<8, 4, QJ>(a, s);
  if (kb == 2) return vb == 2 ? launch_m<2, 2, QJ>(a, s) : launch_m<2, 4, QJ>(a, s);
  if (kb == 3) return vb == 2 ? launch_m<3, 2, QJ>(a, s) : launch_m<3, 4, QJ>(a, s);
  return vb == 2 ? launch_m<4, 2, QJ>(a, s) : launch_m<4, 4, QJ>(a, s);
}

}  // namespace

hipError_t launch_quantize_mfma(const tq_ctx* c, const void* k, const void* v, int64_t num_tokens, int num_kv_heads,
                                const int32_t* slot_mapping, void* pool, int64_t num_blocks, hipStream_t stream) {
  QMArgs a;
  a.k = reinterpret_cast<const uint16_t*>(k);
  a.v = reinterpret_cast<const uint16_t*>(v);
  a.num_tokens = num_tokens;
  a.hkv = num_kv_heads;
  a.slot_mapping = slot_mapping;
  a.slots_total = num_blocks * 16;
  a.pool = reinterpret_cast<uint8_t*>(pool);
  a.rec = c->lay.bytes;
  a.lay = c->lay;
  a.dev = c->dev;
  a.num_tiles = (num_tokens + 15) / 16 * num_kv_heads;
  return c->qjl ? dispatch_m<true>(a, c->kb, c->vb, stream) : dispatch_m<false>(a, c->kb, c->vb, stream);
}

}  // namespace tq
