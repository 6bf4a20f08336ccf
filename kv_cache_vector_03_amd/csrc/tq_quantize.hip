// Fused quantise + pack + paged store for gfx950 (Roadmap §3.1: rotation fused
// with the quantiser in one launch; Hub, technical principle steps 1-5).
//
// Work split: a wave owns a tile of 16 token-heads.  Lane (row = lane/4,
// part = lane%4) holds coordinates [part*E, part*E+E) of its row, E = d/4, so
// the Walsh-Hadamard butterflies run in registers for the strides below E and
// across the 4 lanes of a row (xor 1, xor 2) for the last two.  The QJL
// projection z = S r of the 16 rows is a dense [16 x d] x [d x d] product: it
// runs on v_mfma_f32_16x16x32_f16 with fp16 hi/lo splits of the pre-scaled
// operands (three products per tile: hi*hi + hi*lo + lo*hi), and the sign
// bits come straight out of the accumulator with a wave ballot.
#include <hip/hip_runtime.h>

#include "tq_common.hip.h"
#include "tq_internal.h"

namespace tq {

struct QArgs {
  const void* k;
  const void* v;
  int64_t num_th;  // tokens * kv heads
  int32_t hkv;
  const int32_t* slot_mapping;
  int64_t slots_total;  // 16 * num_blocks
  uint8_t* pool;
  int64_t rec;  // record bytes per (block, head)
  Layout lay;
  DevTables dev;
  int64_t num_tiles;
};

template <int D>
constexpr int kQWaves = D == 128 ? 8 : 4;  // d = 256 needs up to 512 VGPRs per lane

template <int D>
struct QLds {
  static constexpr int KT = D / 32, NT = D / 16;
  static constexpr bool kTilesInLds = (D == 128);
  static constexpr int kRowStride = D + 8;  // halves; padding breaks bank conflicts of the A reads
  static constexpr size_t tiles_bytes = kTilesInLds ? (size_t)NT * KT * 2 * 64 * 8 * 2 : 0;
  static constexpr size_t a_bytes = (size_t)kQWaves<D> * 2 * 16 * kRowStride * 2;
  static constexpr size_t ballot_bytes = (size_t)kQWaves<D> * NT * 4 * 8;
  static constexpr size_t cent_bytes = 1024;  // upper centroids and thresholds (up to 8-bit codes)
  static constexpr size_t total = tiles_bytes + a_bytes + ballot_bytes + cent_bytes;
};

template <bool BF16, int N>
__device__ __forceinline__ void load_row_part(const void* base, int64_t elem_off, float (&x)[N]) {
  if constexpr (BF16) {
    const u32x4* p = reinterpret_cast<const u32x4*>(reinterpret_cast<const uint16_t*>(base) + elem_off);
#pragma unroll
    for (int i = 0; i < N / 8; ++i) {
      u32x4 w = __builtin_nontemporal_load(p + i);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        x[8 * i + 2 * j] = __uint_as_float(w[j] << 16);
        x[8 * i + 2 * j + 1] = __uint_as_float(w[j] & 0xFFFF0000u);
      }
    }
  } else {
    const f32x4* p = reinterpret_cast<const f32x4*>(reinterpret_cast<const float*>(base) + elem_off);
#pragma unroll
    for (int i = 0; i < N / 4; ++i) {
      f32x4 w = __builtin_nontemporal_load(p + i);
#pragma unroll
      for (int j = 0; j < 4; ++j) x[4 * i + j] = w[j];
    }
  }
}

// Lloyd-Max index of a rotated coordinate u for an odd-symmetric codebook
// (c[L-1-k] = -c[k], t[L-2-k] = -t[k], t[H-1] = 0 with H = L/2), from its
// magnitude: cnt = #{upper thresholds t[H..L-2] below |u|}, index = H + cnt
// for u > 0 and H - 1 - cnt otherwise (= cnt ^ H, cnt ^ (H-1)), residual
// u - c[index] = +-(|u| - c[H + cnt]).  Identical to the count #{t < u}
// except where |u| equals a threshold exactly.  tU = t[H..L-2]; s_cU holds
// c[H..L-1] in LDS.
// With 8-bit keys (127 upper thresholds) the count is a binary search over
// the upper thresholds in LDS (s_tU); the register copy tU is unused.
template <int KB>
constexpr int sym_regs() {
  return KB <= 4 ? (1 << KB) / 2 - 1 : 1;
}
// #{t < m} over the 2^k - 1 ascending thresholds t (LDS): k halving steps.
template <int K>
__device__ __forceinline__ uint32_t count_below(float m, const float* t) {
  uint32_t cnt = 0;
#pragma unroll
  for (int s = 1 << (K - 1); s >= 1; s >>= 1) cnt += m > t[cnt + s - 1] ? (uint32_t)s : 0u;
  return cnt;
}
template <int KB>
__device__ __forceinline__ void sym_code(float u, const float (&tU)[sym_regs<KB>()], const float* s_cU,
                                         const float* s_tU, uint32_t& code, float& r) {
  constexpr uint32_t H = (1u << KB) / 2;
  const float m = fabsf(u);
  uint32_t cnt = 0;
  if constexpr (KB <= 4) {
#pragma unroll
    for (int i = 0; i < (int)H - 1; ++i) cnt += m > tU[i] ? 1u : 0u;
  } else {
    cnt = count_below<KB - 1>(m, s_tU);
  }
  const float d = m - s_cU[cnt];
  const bool pos = u > 0.f;
  code = cnt ^ (pos ? H : H - 1u);
  r = pos ? d : -d;
}

// One cross-lane Walsh-Hadamard stage over the 4 lanes of a row (partner =
// lane ^ M): lower lanes x + y, upper lanes y - x, as y + sg * x with
// sg = +-1 (one rounding, identical to the add / subtract).
template <int M>
__device__ __forceinline__ float wht_quad(float x, float sg) {
  constexpr int kCtrl = M == 1 ? 0xB1 : 0x4E;  // quad_perm [1,0,3,2] / [2,3,0,1]
  const float y = __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), kCtrl, 0xF, 0xF, false));
  return __builtin_fmaf(sg, x, y);
}

// Rotated values (Roadmap §4.2, W_O weight absorption): v <- fp32(D2 (H /
// sqrt d) D1 v), the butterflies taken in fp64 so that the one rounding to
// fp32 at the end is the only one (a sum of d fp32 inputs with +-1
// coefficients is exact in fp64 unless their exponents span more than 22
// binades).  Tiled layout: lane (row, part) holds coordinates part * E + e;
// the two highest index bits are the lanes part ^ 1, part ^ 2 of the row.
// m1 / m2: bit e set where D1 / D2 of coordinate part * E + e is -1.
template <int E>
__device__ __forceinline__ void rotate_values_tiled(float (&x)[E], const uint32_t* m1, const uint32_t* m2, int part) {
  double y[E];
#pragma unroll
  for (int e = 0; e < E; ++e) y[e] = ((m1[e / 32] >> (e % 32)) & 1u) ? -(double)x[e] : (double)x[e];
#pragma unroll
  for (int hs = 1; hs < E; hs <<= 1) {
#pragma unroll
    for (int e = 0; e < E; ++e) {
      if ((e & hs) == 0) {
        const double p = y[e], q = y[e + hs];
        y[e] = p + q;
        y[e + hs] = p - q;
      }
    }
  }
#pragma unroll
  for (int m = 1; m <= 2; m <<= 1) {
    const bool upper = (part & m) != 0;
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const double o = __shfl_xor(y[e], m, 64);
      y[e] = upper ? o - y[e] : y[e] + o;
    }
  }
  const double inv = 1.0 / __builtin_sqrt((double)(4 * E));
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const double v = y[e] * inv;
    x[e] = (float)(((m2[e / 32] >> (e % 32)) & 1u) ? -v : v);
  }
}

template <int D, int KB, int VB, bool BF16, bool QJ, bool ROTV>
__global__ __launch_bounds__(kQWaves<D> * 64) void quantize_kernel(QArgs a) {
  constexpr int E = D / 4;
  constexpr int L = 1 << KB;
  constexpr int KT = D / 32, NT = D / 16;
  constexpr int RS = QLds<D>::kRowStride;
  constexpr int SW = E / 32;  // sign-mask words per lane
  extern __shared__ __attribute__((aligned(16))) unsigned char lds[];
  uint16_t* s_tiles = reinterpret_cast<uint16_t*>(lds);
  uint16_t* s_a = reinterpret_cast<uint16_t*>(lds + QLds<D>::tiles_bytes);
  uint64_t* s_ballot = reinterpret_cast<uint64_t*>(lds + QLds<D>::tiles_bytes + QLds<D>::a_bytes);
  float* s_c = reinterpret_cast<float*>(lds + QLds<D>::tiles_bytes + QLds<D>::a_bytes + QLds<D>::ballot_bytes);

  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int row = lane >> 2, part = lane & 3;

  if constexpr (QLds<D>::kTilesInLds && QJ) {
    const u32x4* src = reinterpret_cast<const u32x4*>(a.dev.s_tiles_d2);
    u32x4* dst = reinterpret_cast<u32x4*>(s_tiles);
    constexpr int n16 = (int)(QLds<D>::tiles_bytes / 16);
    for (int i = tid; i < n16; i += kQWaves<D> * 64) dst[i] = src[i];
  }
  // upper half of the (odd-symmetric) codebook: centroids in LDS, thresholds
  // in registers (8-bit codes: in LDS after the centroids)
  constexpr int H = L / 2;
  float* s_tU = s_c + H;
  if (tid < H) s_c[tid] = a.dev.centroids[H + tid];
  float tU[sym_regs<KB>()];
  if constexpr (KB <= 4) {
#pragma unroll
    for (int i = 0; i < H - 1; ++i) tU[i] = a.dev.thresholds[H + i];
  } else {
    tU[0] = 0.f;
    if (tid < H - 1) s_tU[tid] = a.dev.thresholds[H + tid];
  }
  // D1 / D2 signs of this lane's coordinates as bit masks (bit = negative)
  // D1 as sign-bit patterns: fp32 inputs per element (m1), bf16 inputs per
  // packed pair (bits 15 and 31 of each input dword).  D2 acts after the
  // rotation: the kernel works on D2-free coordinates u' (u = D2 u'), whose
  // index under the symmetric codebook is index(u) ^ (L-1) where D2 = -1
  // (applied to the packed code words, pattern m2c) and whose residual is
  // D2 r, projected with the D2-folded tiles.
  constexpr int CW = E * KB / 32;  // code dwords per lane
  uint32_t m1[SW], p1[E / 2], m2c[CW];
#pragma unroll
  for (int w = 0; w < SW; ++w) {
    m1[w] = 0;
#pragma unroll
    for (int b = 0; b < 32; ++b) m1[w] |= (a.dev.signs1[part * E + 32 * w + b] < 0.f ? 1u : 0u) << b;
  }
#pragma unroll
  for (int i = 0; i < E / 2; ++i)
    p1[i] = (a.dev.signs1[part * E + 2 * i] < 0.f ? 0x8000u : 0u) | (a.dev.signs1[part * E + 2 * i + 1] < 0.f ? 0x80000000u : 0u);
#pragma unroll
  for (int i = 0; i < CW; ++i) m2c[i] = 0;
#pragma unroll
  for (int e = 0; e < E; ++e) {
    if (a.dev.signs2[part * E + e] < 0.f) {
      const int bp = e * KB;
      m2c[bp / 32] |= (uint32_t)(L - 1) << (bp % 32);
      if ((bp % 32) + KB > 32) m2c[bp / 32 + 1] |= (uint32_t)(L - 1) >> (32 - bp % 32);
    }
  }
  // D2 of this lane's coordinates as bit masks, for rotated values
  uint32_t m2v[SW];
#pragma unroll
  for (int w = 0; w < SW; ++w) {
    m2v[w] = 0;
    if constexpr (ROTV) {
#pragma unroll
      for (int b = 0; b < 32; ++b) m2v[w] |= (a.dev.signs2[part * E + 32 * w + b] < 0.f ? 1u : 0u) << b;
    }
  }
  const float sg_1 = (part & 1) ? -1.f : 1.f, sg_2 = (part & 2) ? -1.f : 1.f;
  __syncthreads();

  uint16_t* a_hi = s_a + (size_t)wave * 2 * 16 * RS;
  uint16_t* a_lo = a_hi + 16 * RS;
  uint64_t* ballots = s_ballot + (size_t)wave * NT * 4;
  const float inv_sqrt_d = 1.0f / __builtin_sqrtf((float)D);
  const float rscale = (float)(1 << kRScaleLog2);

  // bf16 inputs: the raw K and V dwords of the next tile are requested while
  // the current one is processed (one tile of prefetch in registers)
  const int64_t tstride = (int64_t)gridDim.x * kQWaves<D>;
  constexpr int NR = BF16 ? E / 8 : 1;  // 16-byte pieces of a row part
  auto fetch = [&](int64_t tl, u32x4 (&kd)[NR], u32x4 (&vd)[NR]) {
    const int64_t thx = tl * 16 + row;
    const bool ok = tl < a.num_tiles && thx < a.num_th;
    const int64_t off = ok ? thx * D + part * E : 0;
    const u32x4* pk = reinterpret_cast<const u32x4*>(reinterpret_cast<const uint16_t*>(a.k) + off);
    const u32x4* pv = reinterpret_cast<const u32x4*>(reinterpret_cast<const uint16_t*>(a.v) + off);
#pragma unroll
    for (int i = 0; i < NR; ++i) {
      kd[i] = ok ? __builtin_nontemporal_load(pk + i) : u32x4{0u, 0u, 0u, 0u};
      vd[i] = ok ? __builtin_nontemporal_load(pv + i) : u32x4{0u, 0u, 0u, 0u};
    }
  };
  int64_t tile = (int64_t)blockIdx.x * kQWaves<D> + wave;
  u32x4 kr[NR], vr[NR];
  if constexpr (BF16) fetch(tile, kr, vr);
  for (; tile < a.num_tiles; tile += tstride) {
    const int64_t th = tile * 16 + row;
    const bool valid = th < a.num_th;
    const int64_t t = valid ? th / a.hkv : 0;
    const int h = valid ? (int)(th - t * a.hkv) : 0;
    u32x4 kn[NR], vn[NR];
    if constexpr (BF16) fetch(tile + tstride, kn, vn);

    // ---- key: norm, rotation, Lloyd-Max index, residual
    float x[E];
    if constexpr (BF16) {
      // D1 applied to the packed pairs as they are unpacked
#pragma unroll
      for (int i = 0; i < E / 8; ++i) {
        const u32x4 w = kr[i];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const uint32_t ws = w[j] ^ p1[4 * i + j];
          x[8 * i + 2 * j] = __uint_as_float(ws << 16);
          x[8 * i + 2 * j + 1] = __uint_as_float(ws & 0xFFFF0000u);
        }
      }
    } else {
      if (valid) {
        load_row_part<BF16>(a.k, th * D + part * E, x);
      } else {
#pragma unroll
        for (int e = 0; e < E; ++e) x[e] = 0.f;
      }
#pragma unroll
      for (int e = 0; e < E; ++e) x[e] = __uint_as_float(__float_as_uint(x[e]) ^ (((m1[e / 32] >> (e % 32)) & 1u) << 31));
    }
    // the norm is sign-blind: taken from the D1-flipped values
    float ss = 0.f;
#pragma unroll
    for (int e = 0; e < E; ++e) ss = __builtin_fmaf(x[e], x[e], ss);
    ss = quad_sum_xl(ss);
    const float n = __builtin_sqrtf(ss);
    const bool zero = !(n > 0.f);
#pragma unroll
    for (int hs = 1; hs < E; hs <<= 1) {
#pragma unroll
      for (int e = 0; e < E; ++e) {
        if ((e & hs) == 0) {
          float p = x[e], q = x[e + hs];
          x[e] = p + q;
          x[e + hs] = p - q;
        }
      }
    }
#pragma unroll
    for (int e = 0; e < E; ++e) x[e] = wht_quad<1>(x[e], sg_1);
#pragma unroll
    for (int e = 0; e < E; ++e) x[e] = wht_quad<2>(x[e], sg_2);
    const float inv = zero ? 0.f : inv_sqrt_d / n;
    uint32_t idx[E];
    float r2 = 0.f;
#pragma unroll
    for (int e = 0; e < E; ++e) {
      uint32_t c;
      float r;
      sym_code<KB>(x[e] * inv, tU, s_c, s_tU, c, r);  // D2-free index and residual
      idx[e] = c;
      r = zero ? 0.f : r;
      r2 = __builtin_fmaf(r, r, r2);
      x[e] = r;
    }
    const float gamma = __builtin_sqrtf(quad_sum_xl(r2));

    // ---- stage the scaled residual as fp16 hi/lo rows for the MFMA A operand
    // (MSE-only keys skip the whole sketch)
    if constexpr (QJ) {
#pragma unroll
    for (int e = 0; e < E; e += 2) {
      float v0 = x[e] * rscale, v1 = x[e + 1] * rscale;
      uint16_t h0 = f32_to_f16_bits(v0), h1 = f32_to_f16_bits(v1);
      uint16_t l0 = f32_to_f16_bits(v0 - f16_bits_to_f32(h0)), l1 = f32_to_f16_bits(v1 - f16_bits_to_f32(h1));
      *reinterpret_cast<uint32_t*>(a_hi + row * RS + part * E + e) = (uint32_t)h0 | ((uint32_t)h1 << 16);
      *reinterpret_cast<uint32_t*>(a_lo + row * RS + part * E + e) = (uint32_t)l0 | ((uint32_t)l1 << 16);
    }
    __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): this wave's LDS writes done
    __builtin_amdgcn_wave_barrier();
    f16x8 ahi[KT], alo[KT];
    {
      const int arow = lane & 15, kq = lane >> 4;
#pragma unroll
      for (int kt = 0; kt < KT; ++kt) {
        ahi[kt] = *reinterpret_cast<const f16x8*>(a_hi + arow * RS + 32 * kt + 8 * kq);
        alo[kt] = *reinterpret_cast<const f16x8*>(a_lo + arow * RS + 32 * kt + 8 * kq);
      }
    }
    // ---- z = S r on the matrix cores; sign bits by ballot (two column tiles
    // in flight: independent accumulation chains)
#pragma unroll 2
    for (int nt = 0; nt < NT; ++nt) {
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kt = 0; kt < KT; ++kt) {
        const size_t tb = (((size_t)nt * KT + kt) * 2) * 64 * 8;
        f16x8 bhi, blo;
        if constexpr (QLds<D>::kTilesInLds) {
          bhi = *reinterpret_cast<const f16x8*>(s_tiles + tb + lane * 8);
          blo = *reinterpret_cast<const f16x8*>(s_tiles + tb + 512 + lane * 8);
        } else {
          bhi = *reinterpret_cast<const f16x8*>(a.dev.s_tiles_d2 + tb + lane * 8);
          blo = *reinterpret_cast<const f16x8*>(a.dev.s_tiles_d2 + tb + 512 + lane * 8);
        }
        acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(ahi[kt], bhi, acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(ahi[kt], blo, acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(alo[kt], bhi, acc, 0, 0, 0);
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        uint64_t b = __ballot(acc[r] >= 0.f);
        if (lane == 0) ballots[nt * 4 + r] = b;
      }
    }
    __builtin_amdgcn_s_waitcnt(0xc07f);
    __builtin_amdgcn_wave_barrier();
    }  // QJ

    // ---- pack and store the key record
    const int32_t slot = valid ? a.slot_mapping[t] : -1;
    const bool store = valid && slot >= 0 && (int64_t)slot < a.slots_total;
    uint8_t* base = a.pool + ((int64_t)(slot >> 4) * a.hkv + h) * a.rec;
    const int s = slot & 15;
    {
      uint32_t w[CW];
#pragma unroll
      for (int i = 0; i < CW; ++i) w[i] = 0;
#pragma unroll
      for (int e = 0; e < E; ++e) {
        const int bp = e * KB;
        w[bp / 32] |= idx[e] << (bp % 32);
        if ((bp % 32) + KB > 32) w[bp / 32 + 1] |= idx[e] >> (32 - bp % 32);
      }
      // D2: index(-u') = index(u') ^ (L-1); a zero vector keeps all-zero codes
#pragma unroll
      for (int i = 0; i < CW; ++i) w[i] = zero ? 0u : (w[i] ^ m2c[i]);
      uint32_t qw[SW];
#pragma unroll
      for (int i = 0; i < SW; ++i) {
        if constexpr (!QJ) {
          qw[i] = 0;
          continue;
        }
        uint32_t lo16 = (uint32_t)(ballots[(part * E / 16 + 2 * i) * 4 + (row & 3)] >> (16 * (row >> 2))) & 0xFFFFu;
        uint32_t hi16 = (uint32_t)(ballots[(part * E / 16 + 2 * i + 1) * 4 + (row & 3)] >> (16 * (row >> 2))) & 0xFFFFu;
        qw[i] = zero ? 0u : (lo16 | (hi16 << 16));
      }
      if (store) {
        uint32_t* kc = reinterpret_cast<uint32_t*>(base + a.lay.kcodes + s * (KB * D / 8) + part * (KB * E / 8));
#pragma unroll
        for (int i = 0; i < CW; ++i) kc[i] = w[i];
        if constexpr (QJ) {
          uint32_t* kq = reinterpret_cast<uint32_t*>(base + a.lay.kqjl + s * (D / 8) + part * (E / 8));
#pragma unroll
          for (int i = 0; i < SW; ++i) kq[i] = qw[i];
          if (part == 0) {
            uint32_t meta = (uint32_t)f32_to_f16_bits(zero ? 0.f : n) | ((uint32_t)f32_to_f16_bits(gamma) << 16);
            *reinterpret_cast<uint32_t*>(base + a.lay.kmeta + s * 4) = meta;
          }
        } else if (part == 0) {
          *reinterpret_cast<uint16_t*>(base + a.lay.kmeta + s * 2) = f32_to_f16_bits(zero ? 0.f : n);
        }
      }
    }

    // ---- value: min-max group quantisation of this lane's E channels
    if constexpr (BF16) {
#pragma unroll
      for (int i = 0; i < E / 8; ++i) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          x[8 * i + 2 * j] = __uint_as_float(vr[i][j] << 16);
          x[8 * i + 2 * j + 1] = __uint_as_float(vr[i][j] & 0xFFFF0000u);
        }
      }
    } else if (valid) {
      load_row_part<BF16>(a.v, th * D + part * E, x);
    } else {
#pragma unroll
      for (int e = 0; e < E; ++e) x[e] = 0.f;
    }
    if constexpr (ROTV) rotate_values_tiled<E>(x, m1, m2v, part);
    constexpr int GL = E / 32;  // groups per lane
    constexpr float LV = (float)((1 << VB) - 1);
#pragma unroll
    for (int gl = 0; gl < GL; ++gl) {
      float mn = x[32 * gl], mx = x[32 * gl];
#pragma unroll
      for (int e = 1; e < 32; ++e) {
        mn = fminf(mn, x[32 * gl + e]);
        mx = fmaxf(mx, x[32 * gl + e]);
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
        const float dv = x[32 * gl + e] - zz;
        const float q0 = dv * rs;
        const float t = __builtin_fmaf(__builtin_fmaf(-q0, sc, dv), rs, q0);
        const float q = fminf(fmaxf(__builtin_rintf(t), 0.f), LV);
        vw[(e * VB) / 32] |= (uint32_t)q << ((e * VB) % 32);
      }
      if (store) {
        const int g = part * GL + gl;
#pragma unroll
        for (int i = 0; i < VB; ++i)
          *reinterpret_cast<uint32_t*>(base + a.lay.vcodes + ((g * VB + i) * 16 + s) * 4) = vw[i];
        *reinterpret_cast<uint32_t*>(base + a.lay.vmeta + (g * 16 + s) * 4) = (uint32_t)s16 | ((uint32_t)z16 << 16);
      }
    }
    if constexpr (BF16) {
#pragma unroll
      for (int i = 0; i < NR; ++i) {
        kr[i] = kn[i];
        vr[i] = vn[i];
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Small batches (a decode step stores one token per sequence): one wave per
// token-head, lane l holding coordinates [P l, P l + P), P = d / 64, so every
// elementwise stage is a few instructions per lane instead of d / 4.  The QJL
// projection of a workgroup's four token-heads is one [4 x d] x [d x d]
// product (A rows 0..3) whose column tiles are shared out over the four
// waves; it uses the same fp16 hi/lo operands, tiles and MFMA order as the
// tiled kernel, so its sign bits are identical to the tiled path's.
// ---------------------------------------------------------------------------
constexpr int kRowWaves = 4;
constexpr int64_t kRowPathMaxTokenHeads = 2048;

// P (2 or 4) consecutive elements of a bf16 or fp32 row.
template <bool BF16, int P>
__device__ __forceinline__ void load_few(const void* base, int64_t elem_off, float (&x)[P]) {
  static_assert(P == 2 || P == 4, "row slice");
  if constexpr (BF16) {
    const uint16_t* p = reinterpret_cast<const uint16_t*>(base) + elem_off;
    if constexpr (P == 2) {
      const uint32_t w = *reinterpret_cast<const uint32_t*>(p);
      x[0] = __uint_as_float(w << 16);
      x[1] = __uint_as_float(w & 0xFFFF0000u);
    } else {
      const uint2 w = *reinterpret_cast<const uint2*>(p);
      x[0] = __uint_as_float(w.x << 16);
      x[1] = __uint_as_float(w.x & 0xFFFF0000u);
      x[2] = __uint_as_float(w.y << 16);
      x[3] = __uint_as_float(w.y & 0xFFFF0000u);
    }
  } else {
    const float* p = reinterpret_cast<const float*>(base) + elem_off;
#pragma unroll
    for (int e = 0; e < P; ++e) x[e] = p[e];
  }
}

template <int D, int KB, int VB, bool BF16, bool QJ, bool ROTV>
__global__ __launch_bounds__(kRowWaves * 64) void quantize_rows_kernel(QArgs a) {
  constexpr int P = D / 64;
  constexpr int L = 1 << KB;
  constexpr int KT = D / 32, NT = D / 16;
  constexpr float LV = (float)((1 << VB) - 1);
  __shared__ float s_r[kRowWaves][D];
  __shared__ uint8_t s_code[kRowWaves][D];
  __shared__ uint32_t s_qjl[kRowWaves][D / 32];
  __shared__ float s_cent[L];
  __shared__ float s_thr[KB <= 4 ? 1 : L - 1];  // 8-bit codes: the thresholds, for a binary search
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t th = (int64_t)blockIdx.x * kRowWaves + wave;
  const bool valid = th < a.num_th;  // invalid waves still take part in the barriers
  const int64_t t = valid ? th / a.hkv : 0;
  const int h = valid ? (int)(th - t * a.hkv) : 0;
  const int j0 = lane * P;

  // issue every independent load first
  float x[P], vx[P], sg1[P], sg2[P], thr[KB <= 4 ? L - 1 : 1];
  int32_t slot = -1;
  if (valid) {
    load_few<BF16, P>(a.k, th * D + j0, x);
    load_few<BF16, P>(a.v, th * D + j0, vx);
    slot = a.slot_mapping[t];
  } else {
#pragma unroll
    for (int e = 0; e < P; ++e) x[e] = vx[e] = 0.f;
  }
#pragma unroll
  for (int e = 0; e < P; ++e) {
    sg1[e] = a.dev.signs1[j0 + e];
    sg2[e] = a.dev.signs2[j0 + e];
  }
  if constexpr (KB <= 4) {
#pragma unroll
    for (int i = 0; i < L - 1; ++i) thr[i] = a.dev.thresholds[i];
  } else {
    thr[0] = 0.f;
    for (int i = tid; i < L - 1; i += kRowWaves * 64) s_thr[i] = a.dev.thresholds[i];
  }
  for (int i = tid; i < L; i += kRowWaves * 64) s_cent[i] = a.dev.centroids[i];
  // this wave's projection tiles (column tiles wave, wave + 4, ...): they do
  // not depend on the token, so their round trip overlaps the one above
  constexpr int NTW = NT / kRowWaves;
  f16x8 bhi[NTW][KT], blo[NTW][KT];
  if constexpr (QJ) {
#pragma unroll
    for (int i = 0; i < NTW; ++i) {
#pragma unroll
      for (int kt = 0; kt < KT; ++kt) {
        const size_t tb = ((((size_t)(wave + kRowWaves * i)) * KT + kt) * 2) * 64 * 8;
        bhi[i][kt] = *reinterpret_cast<const f16x8*>(a.dev.s_tiles + tb + lane * 8);
        blo[i][kt] = *reinterpret_cast<const f16x8*>(a.dev.s_tiles + tb + 512 + lane * 8);
      }
    }
  }

  // ---- key: norm, D1, Walsh-Hadamard, 1/sqrt(d) n, D2, Lloyd-Max index, residual
  float ss = 0.f;
#pragma unroll
  for (int e = 0; e < P; ++e) ss = __builtin_fmaf(x[e], x[e], ss);
  const float n = __builtin_sqrtf(wave_sum_xl(ss));
  const bool zero = !(n > 0.f);
#pragma unroll
  for (int e = 0; e < P; ++e) x[e] *= sg1[e];
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
  // the lane-index bits of the transform: butterflies between lanes l, l ^ m
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
  __syncthreads();  // s_cent, s_thr
  const float inv = zero ? 0.f : (1.0f / __builtin_sqrtf((float)D)) / n;
  float r2 = 0.f;
#pragma unroll
  for (int e = 0; e < P; ++e) {
    const float u = x[e] * inv * sg2[e];
    uint32_t c = 0;
    if constexpr (KB <= 4) {
#pragma unroll
      for (int i = 0; i < L - 1; ++i) c += (u > thr[i]) ? 1u : 0u;
    } else {
      c = count_below<KB>(u, s_thr);
    }
    c = zero ? 0u : c;
    const float r = zero ? 0.f : u - s_cent[c];
    r2 = __builtin_fmaf(r, r, r2);
    s_r[wave][j0 + e] = r * (float)(1 << kRScaleLog2);
    s_code[wave][j0 + e] = (uint8_t)c;
  }
  const float gamma = __builtin_sqrtf(wave_sum_xl(r2));
  __syncthreads();  // every wave's residual is in LDS

  // ---- z = S r for the workgroup's token-heads (A rows 0..3); wave w takes
  // column tiles w, w + 4, ...  (skipped for MSE-only keys)
  if constexpr (QJ) {
    const int arow = lane & 15, kq = lane >> 4;
    f16x8 ahi[KT], alo[KT];
#pragma unroll
    for (int kt = 0; kt < KT; ++kt) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float v = arow < kRowWaves ? s_r[arow][32 * kt + 8 * kq + e] : 0.f;
        const uint16_t hb = f32_to_f16_bits(v);
        const uint16_t lb = f32_to_f16_bits(v - f16_bits_to_f32(hb));
        ahi[kt][e] = __builtin_bit_cast(_Float16, hb);
        alo[kt][e] = __builtin_bit_cast(_Float16, lb);
      }
    }
#pragma unroll
    for (int i = 0; i < NTW; ++i) {
      const int nt = wave + kRowWaves * i;
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kt = 0; kt < KT; ++kt) {
        acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(ahi[kt], bhi[i][kt], acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(ahi[kt], blo[i][kt], acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(alo[kt], bhi[i][kt], acc, 0, 0, 0);
      }
      // result row r (token-head r of the group) sits in register r of lanes 0..15
#pragma unroll
      for (int r = 0; r < kRowWaves; ++r) {
        const uint32_t bits = (uint32_t)__ballot(acc[r] >= 0.f) & 0xFFFFu;
        if (lane == 0) reinterpret_cast<uint16_t*>(&s_qjl[r][0])[nt] = (uint16_t)bits;
      }
    }
  }
  __syncthreads();

  // ---- store the key record
  const bool store = valid && slot >= 0 && (int64_t)slot < a.slots_total;
  uint8_t* base = a.pool + ((int64_t)(slot >> 4) * a.hkv + h) * a.rec;
  const int sl = slot & 15;
  if (store) {
    constexpr int CW = D * KB / 32;  // code dwords of the token
    if (lane < CW) {
      // dword `lane` holds bits [32 lane, 32 lane + 32) of the LSB-first code stream
      uint32_t w = 0;
      const int b0 = 32 * lane;
      for (int j = b0 / KB; j * KB < b0 + 32; ++j) {
        const int bp = j * KB - b0;
        const uint32_t c = s_code[wave][j];
        w |= bp >= 0 ? (c << bp) : (c >> (-bp));
      }
      *reinterpret_cast<uint32_t*>(base + a.lay.kcodes + sl * (KB * D / 8) + 4 * lane) = w;
    }
    if constexpr (QJ) {
      if (lane < D / 32)
        *reinterpret_cast<uint32_t*>(base + a.lay.kqjl + sl * (D / 8) + 4 * lane) = zero ? 0u : s_qjl[wave][lane];
      if (lane == 0) {
        const uint32_t meta = (uint32_t)f32_to_f16_bits(zero ? 0.f : n) | ((uint32_t)f32_to_f16_bits(gamma) << 16);
        *reinterpret_cast<uint32_t*>(base + a.lay.kmeta + sl * 4) = meta;
      }
    } else if (lane == 0) {
      *reinterpret_cast<uint16_t*>(base + a.lay.kmeta + sl * 2) = f32_to_f16_bits(zero ? 0.f : n);
    }
  }

  // ---- value: rotation (rotated-value presets; fp64 butterflies as in the
  // tiled kernel, lane bits by shuffles), then min-max quantisation of
  // 32-channel groups (32 / P lanes each)
  if constexpr (ROTV) {
    double y[P];
#pragma unroll
    for (int e = 0; e < P; ++e) y[e] = (double)vx[e] * (double)sg1[e];
#pragma unroll
    for (int hs = 1; hs < P; hs <<= 1) {
#pragma unroll
      for (int e = 0; e < P; ++e) {
        if ((e & hs) == 0) {
          const double p = y[e], q = y[e + hs];
          y[e] = p + q;
          y[e + hs] = p - q;
        }
      }
    }
#pragma unroll
    for (int m = 1; m < 64; m <<= 1) {
      const bool upper = (lane & m) != 0;
#pragma unroll
      for (int e = 0; e < P; ++e) {
        const double o = __shfl_xor(y[e], m, 64);
        y[e] = upper ? o - y[e] : y[e] + o;
      }
    }
    const double inv = 1.0 / __builtin_sqrt((double)D);
#pragma unroll
    for (int e = 0; e < P; ++e) vx[e] = (float)(y[e] * inv * (double)sg2[e]);
  }
  constexpr int GLN = 32 / P;  // lanes per group
  float mn = vx[0], mx = vx[0];
#pragma unroll
  for (int e = 1; e < P; ++e) {
    mn = fminf(mn, vx[e]);
    mx = fmaxf(mx, vx[e]);
  }
  mn = __uint_as_float(group_reduce_xl<GLN>(__float_as_uint(mn), [](uint32_t p, uint32_t q) {
    return __float_as_uint(fminf(__uint_as_float(p), __uint_as_float(q)));
  }));
  mx = __uint_as_float(group_reduce_xl<GLN>(__float_as_uint(mx), [](uint32_t p, uint32_t q) {
    return __float_as_uint(fmaxf(__uint_as_float(p), __uint_as_float(q)));
  }));
  const uint16_t s16 = f32_to_f16_bits((mx - mn) / LV);
  const uint16_t z16 = f32_to_f16_bits(mn);
  const float sc = f16_bits_to_f32(s16), zz = f16_bits_to_f32(z16);
  // this lane's codes placed at their bit positions inside their dword
  constexpr int CPD = 32 / VB;  // codes per dword
  uint32_t part = 0;
#pragma unroll
  for (int e = 0; e < P; ++e) {
    float q = __builtin_rintf((vx[e] - zz) / sc);
    q = fminf(fmaxf(q, 0.f), LV);
    const uint32_t qi = (sc != 0.f) ? (uint32_t)q : 0u;
    part |= qi << (((j0 + e) % CPD) * VB);
  }
  if constexpr (CPD / P > 1) part = group_reduce_xl<CPD / P>(part, [](uint32_t p, uint32_t q) { return p | q; });
  if (store) {
    const int g = j0 / 32;             // group
    const int i = (j0 % 32) / CPD;     // dword of the group
    if ((j0 % CPD) == 0)
      *reinterpret_cast<uint32_t*>(base + a.lay.vcodes + ((g * VB + i) * 16 + sl) * 4) = part;
    if ((j0 % 32) == 0)
      *reinterpret_cast<uint32_t*>(base + a.lay.vmeta + (g * 16 + sl) * 4) = (uint32_t)s16 | ((uint32_t)z16 << 16);
  }
}

template <int D, int KB, int VB, bool BF16, bool QJ, bool ROTV>
static hipError_t launch_rows(const QArgs& a, hipStream_t stream) {
  const int64_t grid = (a.num_th + kRowWaves - 1) / kRowWaves;
  hipLaunchKernelGGL((quantize_rows_kernel<D, KB, VB, BF16, QJ, ROTV>), dim3((unsigned)grid), dim3(kRowWaves * 64), 0, stream, a);
  return hipGetLastError();
}

template <int D, int KB, int VB, bool BF16, bool QJ, bool ROTV>
static hipError_t launch_q(const QArgs& a, hipStream_t stream) {
  auto kern = quantize_kernel<D, KB, VB, BF16, QJ, ROTV>;
  const size_t lds = QLds<D>::total;
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern), hipFuncAttributeMaxDynamicSharedMemorySize,
                                     (int)lds);
  if (e != hipSuccess) return e;
  int dev = 0, cus = 256;
  (void)hipGetDevice(&dev);
  (void)hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  // persistent waves: one workgroup per CU (the LDS footprint allows no more)
  int64_t want = (a.num_tiles + kQWaves<D> - 1) / kQWaves<D>;
  int grid = (int)std::min<int64_t>(want, (int64_t)cus);
  hipLaunchKernelGGL(kern, dim3(grid), dim3(kQWaves<D> * 64), lds, stream, a);
  return hipGetLastError();
}

template <int D, int KB, bool BF16, bool QJ, bool ROTV>
static hipError_t dispatch_vb(const QArgs& a, int vb, hipStream_t s) {
  if (a.num_th <= kRowPathMaxTokenHeads)
    return vb == 2 ? launch_rows<D, KB, 2, BF16, QJ, ROTV>(a, s) : launch_rows<D, KB, 4, BF16, QJ, ROTV>(a, s);
  return vb == 2 ? launch_q<D, KB, 2, BF16, QJ, ROTV>(a, s) : launch_q<D, KB, 4, BF16, QJ, ROTV>(a, s);
}

template <int D, bool BF16, bool QJ, bool ROTV>
static hipError_t dispatch_kb(const QArgs& a, int kb, int vb, hipStream_t s) {
  if constexpr (!QJ)  // 8-bit keys: MSE-only presets (the host rejects them with the QJL sketch)
    if (kb == 8) return dispatch_vb<D, 8, BF16, QJ, ROTV>(a, vb, s);
  switch (kb) {
    case 2: return dispatch_vb<D, 2, BF16, QJ, ROTV>(a, vb, s);
    case 3: return dispatch_vb<D, 3, BF16, QJ, ROTV>(a, vb, s);
    default: return dispatch_vb<D, 4, BF16, QJ, ROTV>(a, vb, s);
  }
}

template <int D, bool BF16>
static hipError_t dispatch_kind(const QArgs& a, bool qjl, bool rotv, int kb, int vb, hipStream_t s) {
  if (rotv)
    return qjl ? dispatch_kb<D, BF16, true, true>(a, kb, vb, s) : dispatch_kb<D, BF16, false, true>(a, kb, vb, s);
  return qjl ? dispatch_kb<D, BF16, true, false>(a, kb, vb, s) : dispatch_kb<D, BF16, false, false>(a, kb, vb, s);
}

hipError_t launch_quantize(const tq_ctx* c, const void* k, const void* v, int in_dtype, int64_t num_tokens,
                           int num_kv_heads, const int32_t* slot_mapping, void* pool, int64_t num_blocks,
                           hipStream_t stream) {
  QArgs a;
  a.k = k;
  a.v = v;
  a.num_th = num_tokens * num_kv_heads;
  a.hkv = num_kv_heads;
  a.slot_mapping = slot_mapping;
  a.slots_total = num_blocks * 16;
  a.pool = reinterpret_cast<uint8_t*>(pool);
  a.rec = c->lay.bytes;
  a.lay = c->lay;
  a.dev = c->dev;
  a.num_tiles = (a.num_th + 15) / 16;
  const bool bf = in_dtype == TQ_DTYPE_BF16;
  // large bf16 batches at head_dim 128 (values not rotated): rotation and
  // projection on the matrix cores
  if (c->d == 128 && bf && !c->rotv && a.num_th > kRowPathMaxTokenHeads)
    return launch_quantize_mfma(c, k, v, num_tokens, num_kv_heads, slot_mapping, pool, num_blocks, stream);
  if (c->d == 128)
    return bf ? dispatch_kind<128, true>(a, c->qjl, c->rotv, c->kb, c->vb, stream)
              : dispatch_kind<128, false>(a, c->qjl, c->rotv, c->kb, c->vb, stream);
  return bf ? dispatch_kind<256, true>(a, c->qjl, c->rotv, c->kb, c->vb, stream)
            : dispatch_kind<256, false>(a, c->qjl, c->rotv, c->kb, c->vb, stream);
}

}  // namespace tq
