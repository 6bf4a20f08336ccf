// Decode attention over the compressed paged cache for gfx950.
//
// Roadmap §3.2 (the vLLM v2 decode design): grouped query heads share one pass
// over a KV head, the query is rotated once and scores come straight from the
// codes through per-query tables, and the softmax runs in the exp2 domain;
// Roadmap §3.1 / §7: the grid is fixed for graph capture and the split
// partials live in a caller-provided workspace; Roadmap §4.4: empty rows and
// empty splits must not produce NaN or divide by zero.
//
// Three launches on one stream:
//   prep    : q~ = D2 (H/sqrt d) D1 q and p = S q~ per (sequence, query head),
//             and the per-preset list of work items (sequence, KV head, split);
//   split   : a persistent grid walks the work items; each 4-wave workgroup
//             streams one chunk of cached tokens (or the recent full-precision
//             window) and leaves (m, l, acc[d]) per query head;
//   combine : log-sum-exp merge of the splits (empty splits contribute 0).
//
// In `split`, a wave consumes 32 tokens (two paged blocks) per step:
//   scores   [G x 16] per block = q~ . c[idx] + p . (2 sigma - 1) on
//            v_mfma_f32_16x16x32_bf16: A = q~ (bf16 hi rows and lo rows stacked
//            in the 16 MFMA rows), B = centroid hi / lo of the packed codes
//            fetched two codes at a time from an LDS pair table, and B = +-1
//            from an LDS byte table for the sign bits;
//   softmax  running max / sum per head in the exp2 domain;
//   values   acc[(group, head)][channel] += (p s)_hi,lo . (128 + q) on the same
//            MFMA, with the zero-points and the +128 bias folded into one
//            per-(group, head) scalar; only the rows of each column's own
//            group are kept at the end.
#include <hip/hip_runtime.h>

#include <cmath>

#include "tq_common.hip.h"
#include "tq_internal.h"

namespace tq {

constexpr int kWaves = 4;
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
  float sm_scale;
  int chunk;
  int splits_cap;
  float* qt;     // [B][Hq][D]
  float* pq;     // [B][Hq][D]
  float* part;   // [B][Hq][splits_cap][D + 2]
  int32_t* work; // [2][B + 1]
  float* out;
  float* scores;
  int scores_stride;
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
// prep: one workgroup of 256 threads per (sequence, query head); the last
// workgroup enumerates the work items (its scan is 256 wide).
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(256) void decode_prep_kernel(DArgs a) {
  __shared__ float s_x[D];
  __shared__ int s_cnt[256];
  const int tid = threadIdx.x;
  const int nq = a.B * a.Hq;
  if ((int)blockIdx.x == nq) {
    // exclusive prefix sums of work items per preset
    for (int pr = 0; pr < 2; ++pr) {
      int carry = 0;
      for (int base = 0; base < a.B; base += 256) {
        int b = base + tid;
        int items = 0;
        if (b < a.B && seq_preset_of(a, b) == pr) items = a.Hkv * seq_splits(a, b);
        s_cnt[tid] = items;
        __syncthreads();
        for (int off = 1; off < 256; off <<= 1) {
          int v = tid >= off ? s_cnt[tid - off] : 0;
          __syncthreads();
          s_cnt[tid] += v;
          __syncthreads();
        }
        if (b < a.B) a.work[pr * (a.B + 1) + b] = carry + s_cnt[tid] - items;
        int tot = s_cnt[255];
        __syncthreads();
        carry += tot;
      }
      if (tid == 0) a.work[pr * (a.B + 1) + a.B] = carry;
      __syncthreads();
    }
    return;
  }
  const int b = blockIdx.x / a.Hq;
  const int pr = seq_preset_of(a, b);
  const DevTables& dv = a.dev[pr];
  const int64_t qoff = (int64_t)blockIdx.x * D;
  for (int j = tid; j < D; j += blockDim.x) {
    float v = a.q_bf16 ? bf16_to_f32(reinterpret_cast<const uint16_t*>(a.q)[qoff + j])
                       : reinterpret_cast<const float*>(a.q)[qoff + j];
    s_x[j] = v * dv.signs1[j];
  }
  __syncthreads();
  for (int h = 1; h < D; h <<= 1) {
    float nv[D / 256 + 1];
    int c = 0;
    for (int j = tid; j < D; j += blockDim.x, ++c) {
      float x = s_x[j], y = s_x[j ^ h];
      nv[c] = (j & h) ? (y - x) : (x + y);
    }
    __syncthreads();
    c = 0;
    for (int j = tid; j < D; j += blockDim.x, ++c) s_x[j] = nv[c];
    __syncthreads();
  }
  const float inv = 1.0f / __builtin_sqrtf((float)D);
  for (int j = tid; j < D; j += blockDim.x) {
    float v = s_x[j] * inv * dv.signs2[j];
    a.qt[qoff + j] = v;
  }
  __syncthreads();
  for (int j = tid; j < D; j += blockDim.x) s_x[j] = s_x[j] * inv * dv.signs2[j];
  __syncthreads();
  for (int i = tid; i < D; i += blockDim.x) {
    const float* row = dv.S + (int64_t)i * D;
    float acc = 0.f;
    for (int j = 0; j < D; ++j) acc = __builtin_fmaf(row[j], s_x[j], acc);
    a.pq[qoff + i] = acc;
  }
}

// ---------------------------------------------------------------------------
// split
// ---------------------------------------------------------------------------
template <int D, int GP>
struct SplitLds {
  static constexpr int kPairBytes = 256 * 8;           // largest pair table (4-bit codes)
  static constexpr int kSignBytes = 256 * 16;           // byte -> 8 bf16 of +-1
  static constexpr int kPBytes = kWaves * GP * 32 * 4;  // per-wave softmax weights
  static constexpr int kMergeBytes = kWaves * GP * D * 4;
  static constexpr int kStatBytes = kWaves * GP * 2 * 4;
  static constexpr int total = kPairBytes + kSignBytes + kPBytes + kMergeBytes + kStatBytes;
};

__device__ __forceinline__ uint32_t bf16_pair_bits(float lo, float hi) {
  return f32_to_bf16_bits(lo) | (f32_to_bf16_bits(hi) << 16);
}

template <int D, int GP, int KB, int VB>
__device__ void split_cached_chunk(const DArgs& a, int pr, int b, int h, int t0, int t1, const uint32_t* s_pair,
                                   const u32x4* s_sign, float* s_p, float* s_merge, float* s_stat,
                                   const bf16x8 (&A1)[D / 32], const bf16x8 (&A3)[D / 32], float* m_out,
                                   float* l_out) {
  constexpr int KT = D / 32;
  constexpr int CS = D / 128;        // value column sets
  constexpr int RT = GP / 4;         // value row tiles per column set
  constexpr int CT = 8;              // value channel tiles per column set
  constexpr int QB = KB * D / 32;    // code bytes per lane quarter
  constexpr int QW = (QB + 3) / 4;   // code dwords per lane quarter
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int tok = lane & 15, kq = lane >> 4;
  const uint8_t* pool = a.pool[pr];
  const Layout lay = a.lay[pr];
  const int64_t rec = a.rec[pr];
  const int32_t* btrow = a.bt + (int64_t)b * a.max_blocks;
  const float kappa = 1.2533141373155003f / (float)D;  // sqrt(pi/2) / d
  float* sp = s_p + wave * GP * 32;

  f32x4 accv[CS][RT][CT];
#pragma unroll
  for (int cs = 0; cs < CS; ++cs)
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
      for (int ct = 0; ct < CT; ++ct) accv[cs][rt][ct] = f32x4{0.f, 0.f, 0.f, 0.f};
  float zacc[CS][RT];
#pragma unroll
  for (int cs = 0; cs < CS; ++cs)
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) zacc[cs][rt] = 0.f;
  float m_run[GP], l_run[GP];
#pragma unroll
  for (int g = 0; g < GP; ++g) {
    m_run[g] = -INFINITY;
    l_run[g] = 0.f;
  }

  const int nsteps = (t1 - t0 + 31) / 32;
  for (int st = wave; st < nsteps; st += kWaves) {
    const int sbase = t0 + st * 32;
    // ------------------------------------------------------------ scores
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      const int blk_tok = sbase + half * 16;
      const int my_tok = blk_tok + tok;
      const bool blk_live = blk_tok < t1;
      int blk = blk_live ? btrow[blk_tok >> 4] : -1;
      const bool blk_ok = blk >= 0 && (int64_t)blk < a.pool_blocks[pr];
      const uint8_t* rbase = pool + ((int64_t)(blk_ok ? blk : 0) * a.Hkv + h) * rec;
      uint32_t cw[QW + 1];
      uint32_t qw[D / 128];
      uint32_t meta = 0;
#pragma unroll
      for (int i = 0; i <= QW; ++i) cw[i] = 0;
#pragma unroll
      for (int i = 0; i < D / 128; ++i) qw[i] = 0;
      if (blk_ok) {
        const uint32_t* cp = reinterpret_cast<const uint32_t*>(rbase + lay.kcodes + tok * (KB * D / 8) + kq * QB);
#pragma unroll
        for (int i = 0; i < QW; ++i) cw[i] = cp[i];
        const uint32_t* qp = reinterpret_cast<const uint32_t*>(rbase + lay.kqjl + tok * (D / 8) + kq * (D / 32));
#pragma unroll
        for (int i = 0; i < D / 128; ++i) qw[i] = qp[i];
        meta = *reinterpret_cast<const uint32_t*>(rbase + lay.kmeta + tok * 4);
      }
      f32x4 am = {0.f, 0.f, 0.f, 0.f}, aq = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kt = 0; kt < KT; ++kt) {
        // 8 codes of this tile: bits [8 kt KB, 8 kt KB + 8 KB) of the quarter
        constexpr int TB = 8 * KB;
        const int bp = kt * TB;
        uint32_t win = bp % 32 == 0 ? cw[bp / 32] : __builtin_amdgcn_alignbit(cw[bp / 32 + 1], cw[bp / 32], bp % 32);
        u32x4 bh, bl;
#pragma unroll
        for (int pi = 0; pi < 4; ++pi) {
          uint32_t pidx = (win >> (2 * KB * pi)) & ((1u << (2 * KB)) - 1u);
          if (KB == 4 && pi == 3) pidx = win >> 24;
          const uint32_t* e = s_pair + 2 * pidx;
          bh[pi] = e[0];
          bl[pi] = e[1];
        }
        am = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A1[kt], __builtin_bit_cast(bf16x8, bh), am, 0, 0, 0);
        am = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A1[kt], __builtin_bit_cast(bf16x8, bl), am, 0, 0, 0);
        const uint32_t sbyte = (qw[kt / 4] >> (8 * (kt % 4))) & 0xFFu;
        u32x4 bq = s_sign[sbyte];
        aq = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A3[kt], __builtin_bit_cast(bf16x8, bq), aq, 0, 0, 0);
      }
      // rows: GP hi rows then GP lo rows -> sum hi + lo
      f32x4 sm, sq;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        if constexpr (GP == 4) {
          auto x = __builtin_amdgcn_permlane16_swap(__float_as_uint(am[r]), __float_as_uint(am[r]), false, false);
          auto y = __builtin_amdgcn_permlane16_swap(__float_as_uint(aq[r]), __float_as_uint(aq[r]), false, false);
          sm[r] = __uint_as_float(x[0]) + __uint_as_float(x[1]);
          sq[r] = __uint_as_float(y[0]) + __uint_as_float(y[1]);
        } else {
          auto x = __builtin_amdgcn_permlane32_swap(__float_as_uint(am[r]), __float_as_uint(am[r]), false, false);
          auto y = __builtin_amdgcn_permlane32_swap(__float_as_uint(aq[r]), __float_as_uint(aq[r]), false, false);
          sm[r] = __uint_as_float(x[0]) + __uint_as_float(x[1]);
          sq[r] = __uint_as_float(y[0]) + __uint_as_float(y[1]);
        }
      }
      const float n = f16_bits_to_f32((uint16_t)(meta & 0xFFFFu));
      const float gm = f16_bits_to_f32((uint16_t)(meta >> 16));
      const bool live = blk_ok && my_tok < t1;
      // lanes 0-15 hold heads 0..3 (and, for GP = 8, lanes 16-31 heads 4..7)
      const int hbase = (GP == 8 && (lane & 16)) ? 4 : 0;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        float est = n * (sm[r] + kappa * gm * sq[r]);
        if (lane < (GP == 8 ? 32 : 16)) {
          const int hh = hbase + r;
          if (hh < a.G && live && a.scores)
            a.scores[((int64_t)b * a.Hq + h * a.G + hh) * a.scores_stride + my_tok] = est;
          sp[hh * 32 + half * 16 + tok] = live ? est * a.logit_scale : -INFINITY;
        }
      }
    }
    __builtin_amdgcn_s_waitcnt(0xc07f);
    __builtin_amdgcn_wave_barrier();
    // ------------------------------------------------------------ softmax
    constexpr int LPH = 64 / GP;   // lanes per head
    constexpr int VPL = 32 / LPH;  // values per lane
    const int mh = lane / LPH, ml = lane % LPH;
    float xs[VPL];
    float mx = -INFINITY;
#pragma unroll
    for (int i = 0; i < VPL; ++i) {
      xs[i] = sp[mh * 32 + ml * VPL + i];
      mx = fmaxf(mx, xs[i]);
    }
    mx = group_max<LPH>(mx);
    float m_new[GP], alpha[GP];
    bool rescale = false;
#pragma unroll
    for (int g = 0; g < GP; ++g) {
      const float mg = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(mx), g * LPH));
      m_new[g] = fmaxf(m_run[g], mg);
      // a head with no live token yet keeps scale 1 (never -inf - -inf)
      alpha[g] = (m_new[g] == -INFINITY) ? 1.f : __builtin_amdgcn_exp2f(m_run[g] - m_new[g]);
      rescale |= alpha[g] != 1.f;
    }
    float mym = m_new[0];
#pragma unroll
    for (int g = 1; g < GP; ++g) mym = (mh == g) ? m_new[g] : mym;
    float lsum = 0.f;
#pragma unroll
    for (int i = 0; i < VPL; ++i) {
      float p = (mym == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(xs[i] - mym);
      lsum += p;
      sp[mh * 32 + ml * VPL + i] = p;
    }
    lsum = group_sum<LPH>(lsum);
#pragma unroll
    for (int g = 0; g < GP; ++g) {
      float lg = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(lsum), g * LPH));
      l_run[g] = l_run[g] * alpha[g] + lg;
      m_run[g] = m_new[g];
    }
    if (rescale) {
#pragma unroll
      for (int cs = 0; cs < CS; ++cs)
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
#pragma unroll
          for (int ct = 0; ct < CT; ++ct)
#pragma unroll
            for (int r = 0; r < 4; ++r) accv[cs][rt][ct][r] *= alpha[4 * rt + r];
          // zacc of row (group, head = 4 rt + (lane & 3))
          float az = alpha[4 * rt];
#pragma unroll
          for (int r = 1; r < 4; ++r) az = ((lane & 3) == r) ? alpha[4 * rt + r] : az;
          zacc[cs][rt] *= az;
        }
    }
    __builtin_amdgcn_s_waitcnt(0xc07f);
    __builtin_amdgcn_wave_barrier();
    // ------------------------------------------------------------ values
    {
      // lane: A row = lane & 15 -> (group 4 cs + row / 4, head 4 rt + row % 4),
      // tokens 8 kq .. 8 kq + 7 of the step (block kq / 2, slots 8 (kq & 1) ..)
      const int vblk_tok = sbase + (kq >> 1) * 16;
      const bool vlive = vblk_tok < t1;
      int vb = vlive ? btrow[vblk_tok >> 4] : -1;
      const bool vok = vb >= 0 && (int64_t)vb < a.pool_blocks[pr];
      const uint8_t* vbase = pool + ((int64_t)(vok ? vb : 0) * a.Hkv + h) * rec;
      const int slot0 = (kq & 1) * 8;
      const int arow = lane & 15;
      float pw[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) pw[e] = 0.f;
#pragma unroll
      for (int cs = 0; cs < CS; ++cs) {
        // value code dwords of this lane's column for 8 slots
        constexpr int WPS = VB == 4 ? 16 : 8;  // dword columns per column set
        const int wcol = cs * WPS + (VB == 4 ? (lane & 15) : (lane & 7));
        uint32_t xv[8];
        if (vok) {
          const u32x4* vp = reinterpret_cast<const u32x4*>(vbase + lay.vcodes + ((int64_t)wcol * 16 + slot0) * 4);
          u32x4 v0 = vp[0], v1 = vp[1];
          xv[0] = v0[0]; xv[1] = v0[1]; xv[2] = v0[2]; xv[3] = v0[3];
          xv[4] = v1[0]; xv[5] = v1[1]; xv[6] = v1[2]; xv[7] = v1[3];
        } else {
#pragma unroll
          for (int e = 0; e < 8; ++e) xv[e] = 0;
        }
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
          const int grp = 4 * cs + (arow >> 2);
          const int hd = 4 * rt + (arow & 3);
          uint32_t sz[8];
          if (vok) {
            const u32x4* mp = reinterpret_cast<const u32x4*>(vbase + lay.vmeta + ((int64_t)grp * 16 + slot0) * 4);
            u32x4 m0 = mp[0], m1 = mp[1];
            sz[0] = m0[0]; sz[1] = m0[1]; sz[2] = m0[2]; sz[3] = m0[3];
            sz[4] = m1[0]; sz[5] = m1[1]; sz[6] = m1[2]; sz[7] = m1[3];
          } else {
#pragma unroll
            for (int e = 0; e < 8; ++e) sz[e] = 0;
          }
          const float* prow = sp + hd * 32 + 8 * kq;
          u32x4 ah, al;
#pragma unroll
          for (int e = 0; e < 8; e += 2) {
            float p0 = prow[e], p1 = prow[e + 1];
            float s0 = f16_bits_to_f32((uint16_t)(sz[e] & 0xFFFFu)), z0 = f16_bits_to_f32((uint16_t)(sz[e] >> 16));
            float s1 = f16_bits_to_f32((uint16_t)(sz[e + 1] & 0xFFFFu)), z1 = f16_bits_to_f32((uint16_t)(sz[e + 1] >> 16));
            float w0 = p0 * s0, w1 = p1 * s1;
            uint32_t h0 = f32_to_bf16_bits(w0), h1 = f32_to_bf16_bits(w1);
            uint32_t l0 = f32_to_bf16_bits(w0 - __uint_as_float(h0 << 16));
            uint32_t l1 = f32_to_bf16_bits(w1 - __uint_as_float(h1 << 16));
            ah[e / 2] = h0 | (h1 << 16);
            al[e / 2] = l0 | (l1 << 16);
            // zero-points, minus exactly the +128 bias the MFMA adds with the
            // split weights (hi + lo is exact in fp32)
            const float a0 = __uint_as_float(h0 << 16) + __uint_as_float(l0 << 16);
            const float a1 = __uint_as_float(h1 << 16) + __uint_as_float(l1 << 16);
            zacc[cs][rt] = __builtin_fmaf(p0, z0, __builtin_fmaf(-128.f, a0, zacc[cs][rt]));
            zacc[cs][rt] = __builtin_fmaf(p1, z1, __builtin_fmaf(-128.f, a1, zacc[cs][rt]));
          }
          const bf16x8 Ah = __builtin_bit_cast(bf16x8, ah), Al = __builtin_bit_cast(bf16x8, al);
#pragma unroll
          for (int ct = 0; ct < CT; ++ct) {
            u32x4 bv;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              if constexpr (VB == 4) {
                const int byte = ct >> 1, par = ct & 1;
                uint32_t y = __builtin_amdgcn_perm(xv[2 * i + 1], xv[2 * i], 0x0C000C00u | (uint32_t)byte | ((uint32_t)(4 + byte) << 16));
                bv[i] = ((par ? (y >> 4) : y) & 0x000F000Fu) | 0x43004300u;
              } else {
                const int bsel = 2 * ((lane & 15) >> 3) + (ct >> 2), sub = ct & 3;
                uint32_t y = __builtin_amdgcn_perm(xv[2 * i + 1], xv[2 * i], 0x0C000C00u | (uint32_t)bsel | ((uint32_t)(4 + bsel) << 16));
                bv[i] = ((y >> (2 * sub)) & 0x00030003u) | 0x43004300u;
              }
            }
            const bf16x8 Bv = __builtin_bit_cast(bf16x8, bv);
            accv[cs][rt][ct] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(Ah, Bv, accv[cs][rt][ct], 0, 0, 0);
            accv[cs][rt][ct] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(Al, Bv, accv[cs][rt][ct], 0, 0, 0);
          }
        }
      }
    }
    __builtin_amdgcn_s_waitcnt(0xc07f);
    __builtin_amdgcn_wave_barrier();
  }

  // ---------------------------------------------------------------- merge
  // zacc: sum the four token quarters (lanes l, l^16, l^32, l^48)
#pragma unroll
  for (int cs = 0; cs < CS; ++cs)
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
      float z = zacc[cs][rt];
      z += __shfl_xor(z, 16, 64);
      z += __shfl_xor(z, 32, 64);
      zacc[cs][rt] = z;
    }
  float* mw = s_merge + wave * GP * D;
  // each wave writes its own un-normalised acc[head][channel]: output row
  // (group l/16, head 4 rt + r) of column j is kept where the column's channel
  // belongs to that group
#pragma unroll
  for (int cs = 0; cs < CS; ++cs)
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
      for (int ct = 0; ct < CT; ++ct)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int j = lane & 15, gl = lane >> 4;
          int ch;
          if constexpr (VB == 4)
            ch = 128 * cs + 8 * j + 2 * (ct >> 1) + (ct & 1);
          else
            ch = 128 * cs + 16 * (j & 7) + 4 * (2 * (j >> 3) + (ct >> 2)) + (ct & 3);
          const int grp_local = (ch >> 5) - 4 * cs;
          // zero-point / bias term of row (group, head) sits in the lanes whose
          // A row is 4 grp_local + r
          const float zz = __shfl(zacc[cs][rt], 4 * grp_local + r, 64);
          if (grp_local == gl) mw[(4 * rt + r) * D + ch] = accv[cs][rt][ct][r] + zz;
        }
  if (lane == 0) {
#pragma unroll
    for (int g = 0; g < GP; ++g) {
      s_stat[(wave * GP + g) * 2] = m_run[g];
      s_stat[(wave * GP + g) * 2 + 1] = l_run[g];
    }
  }
  __syncthreads();
  // combine the four waves; results for head g in m_out[g], l_out[g] and s_merge[0][g][:]
  const int tid = threadIdx.x;
  for (int idx = tid; idx < GP * D; idx += kWaves * 64) {
    const int g = idx / D;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) M = fmaxf(M, s_stat[(w * GP + g) * 2]);
    float acc = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      float lw = s_stat[(w * GP + g) * 2 + 1];
      float f = lw > 0.f ? __builtin_amdgcn_exp2f(s_stat[(w * GP + g) * 2] - M) : 0.f;
      acc += f * s_merge[w * GP * D + idx];
    }
    s_merge[idx] = acc;  // wave 0's slot is consumed in place (read above before write by this thread only)
  }
  if (tid < GP) {
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) M = fmaxf(M, s_stat[(w * GP + tid) * 2]);
    float L = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      float lw = s_stat[(w * GP + tid) * 2 + 1];
      L += lw > 0.f ? lw * __builtin_amdgcn_exp2f(s_stat[(w * GP + tid) * 2] - M) : 0.f;
    }
    m_out[tid] = L > 0.f ? M : -INFINITY;
    l_out[tid] = L;
  }
  __syncthreads();
}

// Recent full-precision window: exact scores <q, k> with the unrotated query
// and bf16 keys, bf16 values.  One token per lane for the scores, one channel
// per lane for the values (the window is small next to the cache).
template <int D, int GP>
__device__ void split_recent(const DArgs& a, int b, int h, int R, float* s_p, float* s_merge, float* m_out,
                             float* l_out) {
  const int tid = threadIdx.x;
  const uint16_t* kb = a.rk + (((int64_t)b * a.Hkv + h) * a.W) * D;
  const uint16_t* vb = a.rv + (((int64_t)b * a.Hkv + h) * a.W) * D;
  // s_p reused as [GP][W] logits (W <= 4096 fits in the merge area instead when large)
  float* lg = s_merge;  // [GP][R] logits, then weights; R <= W
  for (int idx = tid; idx < a.G * R; idx += kWaves * 64) {
    const int g = idx / R, t = idx % R;
    const int64_t qoff = ((int64_t)b * a.Hq + h * a.G + g) * D;
    float acc = 0.f;
    for (int j = 0; j < D; ++j) {
      float qv = a.q_bf16 ? bf16_to_f32(reinterpret_cast<const uint16_t*>(a.q)[qoff + j])
                          : reinterpret_cast<const float*>(a.q)[qoff + j];
      acc = __builtin_fmaf(qv, bf16_to_f32(kb[(int64_t)t * D + j]), acc);
    }
    if (a.scores) a.scores[((int64_t)b * a.Hq + h * a.G + g) * a.scores_stride + seq_cached(a, b) + t] = acc;
    lg[g * R + t] = acc * a.logit_scale;
  }
  __syncthreads();
  if (tid < a.G) {
    float M = -INFINITY;
    for (int t = 0; t < R; ++t) M = fmaxf(M, lg[tid * R + t]);
    float L = 0.f;
    for (int t = 0; t < R; ++t) {
      float p = __builtin_amdgcn_exp2f(lg[tid * R + t] - M);
      lg[tid * R + t] = p;
      L += p;
    }
    m_out[tid] = M;
    l_out[tid] = L;
  }
  __syncthreads();
  // acc[g][c] into s_p scratch area (GP * D floats available after the merge area)
  float* accs = s_merge + GP * a.W;
  for (int idx = tid; idx < a.G * D; idx += kWaves * 64) {
    const int g = idx / D, c = idx % D;
    float acc = 0.f;
    for (int t = 0; t < R; ++t) acc = __builtin_fmaf(lg[g * R + t], bf16_to_f32(vb[(int64_t)t * D + c]), acc);
    accs[idx] = acc;
  }
  __syncthreads();
  for (int idx = tid; idx < a.G * D; idx += kWaves * 64) s_merge[idx] = accs[idx];
  __syncthreads();
}

template <int D, int GP, int KB, int VB>
__global__ __launch_bounds__(kWaves * 64) void decode_split_kernel(DArgs a, int pr) {
  constexpr int KT = D / 32;
  extern __shared__ __attribute__((aligned(16))) unsigned char lds[];
  uint32_t* s_pair = reinterpret_cast<uint32_t*>(lds);
  u32x4* s_sign = reinterpret_cast<u32x4*>(lds + SplitLds<D, GP>::kPairBytes);
  float* s_p = reinterpret_cast<float*>(lds + SplitLds<D, GP>::kPairBytes + SplitLds<D, GP>::kSignBytes);
  float* s_merge = s_p + kWaves * GP * 32;
  float* s_stat = s_merge + kWaves * GP * D;
  __shared__ float s_m[kMaxG], s_l[kMaxG];
  const int tid = threadIdx.x, lane = tid & 63;

  // tables: centroid pairs of this preset, +-1 patterns of sign bytes
  const DevTables& dv = a.dev[pr];
  for (int i = tid; i < (1 << (2 * KB)) * 2; i += kWaves * 64) s_pair[i] = dv.pair_lut[i];
  for (int v = tid; v < 256; v += kWaves * 64) {
    u32x4 w;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      uint32_t lo = ((v >> (2 * i)) & 1) ? 0x3F80u : 0xBF80u;
      uint32_t hi = ((v >> (2 * i + 1)) & 1) ? 0x3F80u : 0xBF80u;
      w[i] = lo | (hi << 16);
    }
    s_sign[v] = w;
  }
  __syncthreads();

  const int32_t* cum = a.work + pr * (a.B + 1);
  const int total = cum[a.B];  // written by the prep launch on the same stream
  for (int item = blockIdx.x; item < total; item += gridDim.x) {
    // find the sequence: largest b with cum[b] <= item
    int lo = 0, hi = a.B - 1;
    while (lo < hi) {
      int mid = (lo + hi + 1) >> 1;
      if (cum[mid] <= item) lo = mid; else hi = mid - 1;
    }
    const int b = lo;
    const int local = item - cum[b];
    const int nsp = seq_splits(a, b);
    if (nsp <= 0 || local < 0 || local >= nsp * a.Hkv) break;  // inconsistent work list: stop
    const int h = local / nsp, c = local % nsp;
    const int Lc = seq_cached(a, b);
    const int nq_chunks = (Lc + a.chunk - 1) / a.chunk;

    if (c < nq_chunks) {
      // A operands: rows 0..GP-1 = hi parts of head rows, GP..2GP-1 = lo parts
      bf16x8 A1[KT], A3[KT];
      {
        const int arow = lane & 15, kq = lane >> 4;
        const int g = arow % GP;
        const bool is_lo = arow >= GP;
        const bool used = arow < 2 * GP && g < a.G;
        const int64_t qo = ((int64_t)b * a.Hq + h * a.G + (used ? g : 0)) * D;
#pragma unroll
        for (int kt = 0; kt < KT; ++kt) {
          u32x4 w1, w3;
#pragma unroll
          for (int e = 0; e < 8; e += 2) {
            const int j = kq * (D / 4) + 8 * kt + e;
            float x0 = used ? a.qt[qo + j] : 0.f, x1 = used ? a.qt[qo + j + 1] : 0.f;
            float y0 = used ? a.pq[qo + j] : 0.f, y1 = used ? a.pq[qo + j + 1] : 0.f;
            uint32_t hx0 = f32_to_bf16_bits(x0), hx1 = f32_to_bf16_bits(x1);
            uint32_t hy0 = f32_to_bf16_bits(y0), hy1 = f32_to_bf16_bits(y1);
            if (is_lo) {
              hx0 = f32_to_bf16_bits(x0 - __uint_as_float(hx0 << 16));
              hx1 = f32_to_bf16_bits(x1 - __uint_as_float(hx1 << 16));
              hy0 = f32_to_bf16_bits(y0 - __uint_as_float(hy0 << 16));
              hy1 = f32_to_bf16_bits(y1 - __uint_as_float(hy1 << 16));
            }
            w1[e / 2] = hx0 | (hx1 << 16);
            w3[e / 2] = hy0 | (hy1 << 16);
          }
          A1[kt] = __builtin_bit_cast(bf16x8, w1);
          A3[kt] = __builtin_bit_cast(bf16x8, w3);
        }
      }
      const int t0 = c * a.chunk;
      const int t1 = min(t0 + a.chunk, Lc);
      split_cached_chunk<D, GP, KB, VB>(a, pr, b, h, t0, t1, s_pair, s_sign, s_p, s_merge, s_stat, A1, A3, s_m, s_l);
    } else {
      split_recent<D, GP>(a, b, h, seq_recent(a, b), s_p, s_merge, s_m, s_l);
    }
    // write the partial: (m, l, acc[D]) per query head of this KV head
    for (int idx = tid; idx < a.G * (D + 2); idx += kWaves * 64) {
      const int g = idx / (D + 2), k = idx % (D + 2);
      float v = k == 0 ? s_m[g] : (k == 1 ? s_l[g] : s_merge[g * D + (k - 2)]);
      a.part[(((int64_t)b * a.Hq + h * a.G + g) * a.splits_cap + c) * (D + 2) + k] = v;
    }
    __syncthreads();
  }
}

// ---------------------------------------------------------------------------
// combine: one workgroup of D threads per (sequence, query head)
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(256) void decode_combine_kernel(DArgs a) {
  const int bh = blockIdx.x;
  const int b = bh / a.Hq;
  const int ns = seq_splits(a, b);
  const float* pp = a.part + (int64_t)bh * a.splits_cap * (D + 2);
  float M = -INFINITY;
  for (int s = 0; s < ns; ++s) {
    if (pp[s * (D + 2) + 1] > 0.f) M = fmaxf(M, pp[s * (D + 2)]);
  }
  float L = 0.f;
  for (int s = 0; s < ns; ++s) {
    float l = pp[s * (D + 2) + 1];
    if (l > 0.f) L += l * __builtin_amdgcn_exp2f(pp[s * (D + 2)] - M);
  }
  for (int c = threadIdx.x; c < D; c += blockDim.x) {
    float acc = 0.f;
    for (int s = 0; s < ns; ++s) {
      float l = pp[s * (D + 2) + 1];
      if (l > 0.f) acc += __builtin_amdgcn_exp2f(pp[s * (D + 2)] - M) * pp[s * (D + 2) + 2 + c];
    }
    a.out[(int64_t)bh * D + c] = L > 0.f ? acc / L : 0.f;
  }
}

// ---------------------------------------------------------------------------
template <int D, int GP, int KB, int VB>
static hipError_t launch_split(const DArgs& a, int pr, hipStream_t s) {
  auto kern = decode_split_kernel<D, GP, KB, VB>;
  size_t lds = SplitLds<D, GP>::total;
  size_t recent_need = (size_t)(GP * a.W + GP * D) * 4 + SplitLds<D, GP>::kPairBytes + SplitLds<D, GP>::kSignBytes +
                       SplitLds<D, GP>::kPBytes + SplitLds<D, GP>::kStatBytes;
  if (recent_need > lds) lds = recent_need;
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern), hipFuncAttributeMaxDynamicSharedMemorySize,
                                     (int)lds);
  if (e != hipSuccess) return e;
  int dev = 0, cus = 256;
  (void)hipGetDevice(&dev);
  (void)hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  hipLaunchKernelGGL(kern, dim3(cus * 8), dim3(kWaves * 64), lds, s, a, pr);
  return hipGetLastError();
}

template <int D, int GP>
static hipError_t dispatch_preset(const DArgs& a, int pr, int kb, int vb, hipStream_t s) {
  if (kb == 2) return vb == 2 ? launch_split<D, GP, 2, 2>(a, pr, s) : launch_split<D, GP, 2, 4>(a, pr, s);
  if (kb == 3) return vb == 2 ? launch_split<D, GP, 3, 2>(a, pr, s) : launch_split<D, GP, 3, 4>(a, pr, s);
  return vb == 2 ? launch_split<D, GP, 4, 2>(a, pr, s) : launch_split<D, GP, 4, 4>(a, pr, s);
}

template <int D>
static hipError_t launch_all(const DArgs& a, const tq_decode_args* args, hipStream_t s) {
  hipLaunchKernelGGL(decode_prep_kernel<D>, dim3(a.B * a.Hq + 1), dim3(256), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  for (int pr = 0; pr < args->num_presets; ++pr) {
    const tq_ctx* c = args->ctx[pr];
    e = a.G <= 4 ? dispatch_preset<D, 4>(a, pr, c->kb, c->vb, s) : dispatch_preset<D, 8>(a, pr, c->kb, c->vb, s);
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(decode_combine_kernel<D>, dim3(a.B * a.Hq), dim3(D < 256 ? D : 256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_decode(const tq_decode_args* args, const DecodePlan& plan, hipStream_t stream) {
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
  a.chunk = args->chunk_tokens;
  a.splits_cap = plan.num_splits_max;
  char* ws = reinterpret_cast<char*>(args->workspace);
  a.qt = reinterpret_cast<float*>(ws + plan.off_qt);
  a.pq = reinterpret_cast<float*>(ws + plan.off_p);
  a.part = reinterpret_cast<float*>(ws + plan.off_part);
  a.work = reinterpret_cast<int32_t*>(ws + plan.off_work);
  a.out = args->out;
  a.scores = args->scores_out;
  a.scores_stride = args->scores_stride;
  return plan.d == 128 ? launch_all<128>(a, args, stream) : launch_all<256>(a, args, stream);
}

}  // namespace tq
