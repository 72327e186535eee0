// Weight-streaming products for few rows (decode): C[m, n] = epi(sum_s A_s[row(m)] . B_s[n]).
//
// With a handful of rows per product (a decode batch, or the few tokens an
// expert receives from it) the work is bound by reading the [N, K] weights
// from HBM once. Each wavefront owns a slab of 16 output columns and streams
// its 16 weight rows straight from global memory into MFMA operand registers
// (16 bytes per lane per load; no LDS and no barriers), so many independent
// waves per CU keep enough bytes in flight. The rows' activations are loaded
// the same way; they are few and stay in the caches.
//
// v_mfma_f32_16x16x32_bf16 takes the weight fragment as first operand: lane l
// ends up with output row m = l % 16 of its m-tile and the four columns
// n0 + 4*(l / 16) + 0..3.
//
// Dense products (fc1 / shared up, fc2 + shared down, router) split K over
// KSPLIT waves per column block; each writes its fp32 partial and skinny_reduce sums
// the partials in a fixed order and applies the epilogue, so results do not
// depend on timing. Grouped products (experts) need no split: a slab of one
// expert covers its rows, and there are E x N/16 slabs. Their weights may also
// come as MXFP8 or MXFP4 (E4M3 / E2M1 codes with a power-of-two scale per 32 k), decoded to
// bf16 in registers on the way to the MFMA: half the bytes of bf16 weights.
#include "kernels.h"

namespace moe {

typedef float f32x4v __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2v __attribute__((ext_vector_type(2)));

// 8 E4M3 codes (k order, lowest byte first) times the block scale 2^(s - 127)
// as one bf16 MFMA operand: v_cvt_scalef32_pk_bf16_fp8 decodes two codes and
// scales them; the products are bf16 values, so nothing is rounded.
__device__ __forceinline__ u32x4 mx_decode8(u32x2 c, uint32_t s) {
  const float sc = __uint_as_float(s == 0 ? 0x00400000u : (s << 23));
  const bf16x2v p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(c.x, sc, false);
  const bf16x2v p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(c.x, sc, true);
  const bf16x2v p2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(c.y, sc, false);
  const bf16x2v p3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(c.y, sc, true);
  return u32x4{__builtin_bit_cast(uint32_t, p0), __builtin_bit_cast(uint32_t, p1), __builtin_bit_cast(uint32_t, p2),
               __builtin_bit_cast(uint32_t, p3)};
}

// weight bytes each lane keeps in flight (the loop unroll follows from it)
#ifndef MOE_SKINNY_DENSE64
#define MOE_SKINNY_DENSE64 1
#endif
#ifndef MOE_SKINNY_INFLIGHT
#define MOE_SKINNY_INFLIGHT 128
#endif
#ifndef MOE_SKINNY_MX_INFLIGHT
#define MOE_SKINNY_MX_INFLIGHT 256
#endif
// Grouped MX products with wide outputs take 4 slabs per wave (one set of
// activation fragments serves 4 weight fragments) when that still leaves this
// many waves. Measured on a 64-token decode: faster for the expert up product
// (N = 5120) in both formats, for N = 2048 faster with MXFP4 (0.92 -> 0.70 ms)
// and slower with MXFP8 (1.03 -> 1.19 ms); slower with bf16 weights.
#ifndef MOE_SKINNY_WIDE_WAVES
#define MOE_SKINNY_WIDE_WAVES 4096
#endif
#ifndef MOE_SKINNY_WIDE_MIN_N
#define MOE_SKINNY_WIDE_MIN_N 4096       // MXFP8
#endif
#ifndef MOE_SKINNY_WIDE_MIN_N4
#define MOE_SKINNY_WIDE_MIN_N4 2048      // MXFP4
#endif
constexpr int64_t kGroupedWideWaves = MOE_SKINNY_WIDE_WAVES;

// Four results rounded to bf16, each added to its bf16 residual in fp32 (exact)
// and rounded once more: the block's residual add.
__device__ __forceinline__ u32x2 add_residual_bf16x4(const f32x4v& v, const uint16_t* res) {
  const u32x2 r = *reinterpret_cast<const u32x2*>(res);
  float o[4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
    o[i] = bf16_bits_to_f32(f32_to_bf16_bits(v[i])) + bf16_bits_to_f32((r[i / 2] >> (16 * (i % 2))) & 0xFFFFu);
  return u32x2{pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3])};
}

// 8 fp32 weights (a: k 0..3, b: k 4..7) split exactly into three bf16x8 MFMA
// operands: hi = bf16(w), mid = bf16(w - hi), lo = bf16(w - hi - mid) (each
// difference is exact, and the three parts sum to w).
__device__ __forceinline__ void split3_bf16x8(const u32x4 a, const u32x4 b, u32x4 (&part)[3]) {
  float r[8];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    r[i] = __uint_as_float(a[i]);
    r[4 + i] = __uint_as_float(b[i]);
  }
#pragma unroll
  for (int q = 0; q < 3; ++q) {
    uint32_t bits[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      bits[i] = f32_to_bf16_bits(r[i]);
      r[i] -= bf16_bits_to_f32(bits[i]);
    }
    part[q] = u32x4{bits[0] | (bits[1] << 16), bits[2] | (bits[3] << 16), bits[4] | (bits[5] << 16),
                    bits[6] | (bits[7] << 16)};
  }
}

// 8 E2M1 codes (k order, lowest nibble first) times the block scale as one
// bf16 MFMA operand: v_cvt_scalef32_pk_bf16_fp4 decodes the two codes of a
// byte and scales them, exactly.
__device__ __forceinline__ u32x4 mx4_decode8(uint32_t c, uint32_t s) {
  const float sc = __uint_as_float(s == 0 ? 0x00400000u : (s << 23));
  return u32x4{__builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(c, sc, 0)),
               __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(c, sc, 1)),
               __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(c, sc, 2)),
               __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(c, sc, 3))};
}

int skinny_slabs_per_wave(const SkinnyProblem& P) {
  if (P.offsets == nullptr) return P.M > 16 ? 4 : 1;
  const int min_n = P.mx_fp4 ? MOE_SKINNY_WIDE_MIN_N4 : MOE_SKINNY_WIDE_MIN_N;
  const bool wide =
      P.mx_codes != nullptr && P.N >= min_n && (int64_t)P.groups * ((P.N + 63) / 64) >= kGroupedWideWaves;
  return wide ? 4 : 1;
}

// MT m-tiles of 16 rows and NS slabs of 16 columns per wave. The k axis goes
// in 64-deep steps of two 16x16x32 MFMAs; in each step lane group g = lane/16
// holds k = 16g .. 16g+15 of the step (the first MFMA takes its low 8, the
// second its high 8), so a lane's weights of a step are 16 consecutive
// elements: two 16-byte loads of bf16, one 16-byte (MXFP8) or 8-byte (MXFP4)
// load of codes plus the one scale byte they share, or four 16-byte loads of fp32 weights (the
// router's), each split exactly into three bf16 parts hi + mid + lo that take
// one MFMA each. The activations are loaded in the same k order, so the
// products are unchanged; per step the wave issues MT*NS*2 MFMAs (three times
// that for fp32 weights) and reads the activations once per NS weight
// fragments.
template <int MT, int NS, int UNROLL, int BMODE>
__device__ __forceinline__ void skinny_tile(const SkinnyProblem& P, int n_first, int rows, int row0,
                                            const int32_t* gather, int64_t b_base, int k_begin, int k_end,
                                            int out_row0, float* partial, int lane, int epi,
                                            f32x4v* acc_out = nullptr) {
  // rows of the MT m-tiles this lane loads (clamped: padding lanes re-read a valid row)
  int64_t arow[MT];
#pragma unroll
  for (int t = 0; t < MT; ++t) {
    const int m = min(t * 16 + (lane & 15), rows - 1);
    arow[t] = gather ? (int64_t)gather[row0 + m] : (int64_t)(row0 + m);
  }
  int nrow[NS];
#pragma unroll
  for (int j = 0; j < NS; ++j) nrow[j] = min(n_first + j * 16 + (lane & 15), P.Nb - 1);
  const int kl = (lane >> 4) * 16;         // this lane's 16 k values within a 64-wide step
  f32x4v acc[NS][MT];
#pragma unroll
  for (int j = 0; j < NS; ++j)
#pragma unroll
    for (int t = 0; t < MT; ++t) acc[j][t] = f32x4v{0.f, 0.f, 0.f, 0.f};

  constexpr bool MX = BMODE == kSkinnyMx, MX4 = BMODE == kSkinnyMx4, F32 = BMODE == kSkinnyF32;
  // what one lane loads for one slab in one step: bf16 weights (w[0..1]), MX codes
  // (w[0], decoded at use) and their block scale, or fp32 weights (w[0..3])
  struct BRaw {
    u32x4 w[4];
    uint32_t s;
  };

  // walk the K segments; k indices are global over the concatenated segments
  int seg_k0 = 0;
  for (int s = 0; s < P.nseg; ++s) {
    const KSeg& S = P.seg[s];
    const int lo = max(k_begin, seg_k0), hi = min(k_end, seg_k0 + S.K);
    if (lo < hi) {
      const uint16_t* bp[NS];
      const uint8_t* cp[NS];                 // MX: codes and the block scale of this lane's k
      const uint8_t* sp[NS];
      const uint8_t* sq[NS];                 // MX: the scale row at the segment's first k
      const float* fp[NS];                   // fp32 weights
#pragma unroll
      for (int j = 0; j < NS; ++j) {
        const int64_t e0 = b_base + (int64_t)nrow[j] * S.ldb + (lo - seg_k0) + kl;
        if constexpr (MX || MX4) {
          cp[j] = P.mx_codes + (MX4 ? e0 / 2 : e0);
          sq[j] = P.mx_scales + b_base / 32 + (int64_t)nrow[j] * (S.ldb / 32) + (lo - seg_k0) / 32;
          sp[j] = sq[j] + kl / 32;
        } else if constexpr (F32) {
          fp[j] = P.f32_b + e0;
        } else {
          bp[j] = S.B + e0;
        }
      }
      auto load_b = [&](int j, int st, bool scale = true) -> BRaw {
        BRaw r;
        if constexpr (MX) {
          r.w[0] = *reinterpret_cast<const u32x4*>(cp[j] + st * 64);
          if (scale) r.s = sp[j][st * 2];
        } else if constexpr (MX4) {
          const u32x2 c = *reinterpret_cast<const u32x2*>(cp[j] + st * 32);
          r.w[0] = u32x4{c.x, c.y, 0u, 0u};
          if (scale) r.s = sp[j][st * 2];
        } else if constexpr (F32) {
#pragma unroll
          for (int q = 0; q < 4; ++q) r.w[q] = *reinterpret_cast<const u32x4*>(fp[j] + st * 64 + 4 * q);
        } else {
          r.w[0] = *reinterpret_cast<const u32x4*>(bp[j] + st * 64);
          r.w[1] = *reinterpret_cast<const u32x4*>(bp[j] + st * 64 + 8);
        }
        return r;
      };
      const uint16_t* ap[MT];
#pragma unroll
      for (int t = 0; t < MT; ++t) ap[t] = S.A + arow[t] * S.lda + (lo - seg_k0) + kl;
      auto mfma_step = [&](const BRaw (&b)[NS], const u32x4 (&a0)[MT], const u32x4 (&a1)[MT]) {
#pragma unroll
        for (int j = 0; j < NS; ++j) {
          if constexpr (F32) {
#pragma unroll
            for (int h = 0; h < 2; ++h) {
              u32x4 part[3];
              split3_bf16x8(b[j].w[2 * h], b[j].w[2 * h + 1], part);
#pragma unroll
              for (int q = 0; q < 3; ++q)
#pragma unroll
                for (int t = 0; t < MT; ++t)
                  acc[j][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                      __builtin_bit_cast(bf16x8, part[q]), __builtin_bit_cast(bf16x8, h ? a1[t] : a0[t]), acc[j][t],
                      0, 0, 0);
            }
          } else {
            u32x4 w0 = b[j].w[0], w1 = b[j].w[1];
            if constexpr (MX) {
              w1 = mx_decode8(u32x2{b[j].w[0].z, b[j].w[0].w}, b[j].s);
              w0 = mx_decode8(u32x2{b[j].w[0].x, b[j].w[0].y}, b[j].s);
            } else if constexpr (MX4) {
              w1 = mx4_decode8(b[j].w[0].y, b[j].s);
              w0 = mx4_decode8(b[j].w[0].x, b[j].s);
            }
#pragma unroll
            for (int t = 0; t < MT; ++t) {
              acc[j][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, w0),
                                                                  __builtin_bit_cast(bf16x8, a0[t]), acc[j][t], 0, 0,
                                                                  0);
              acc[j][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, w1),
                                                                  __builtin_bit_cast(bf16x8, a1[t]), acc[j][t], 0, 0,
                                                                  0);
            }
          }
        }
      };
      const int nsteps = (hi - lo) / 64;
      // MX scales of UNROLL steps in one load: a step takes two scale bytes of
      // a row (lane group g the (g >> 1)-th), so a row's scales of the UNROLL
      // steps are 2 * UNROLL consecutive bytes, shared by the lane's four lane
      // groups; one byte load per step instead touched the 16 rows' lines
      // every step. Used when those bytes are aligned for the wide load.
      constexpr int SB = 2 * UNROLL;           // scale bytes of UNROLL steps
      constexpr bool kScaleBlock = (MX || MX4) && (UNROLL == 4 || UNROLL == 8);
      bool sblock = false;
      if constexpr (kScaleBlock) {
        bool al = (S.ldb / 32) % SB == 0 && ((lo - seg_k0) / 32) % SB == 0 && (b_base / 32) % SB == 0 &&
                  (reinterpret_cast<uintptr_t>(P.mx_scales) & (SB - 1)) == 0;
        sblock = al;
      }
      const int sh = (lane >> 5) * 8;          // lane group g = lane / 16 takes byte g >> 1 of a step's pair
      int st = 0;
      for (; st + UNROLL <= nsteps; st += UNROLL) {
        BRaw bv[UNROLL][NS];
        u32x4 a0[UNROLL][MT], a1[UNROLL][MT];
        if (kScaleBlock && sblock) {
#pragma unroll
          for (int u = 0; u < UNROLL; ++u)
#pragma unroll
            for (int j = 0; j < NS; ++j) bv[u][j] = load_b(j, st + u, false);
#pragma unroll
          for (int j = 0; j < NS; ++j) {
            uint32_t w[4];
            if constexpr (SB == 16) {
              const u32x4 v = *reinterpret_cast<const u32x4*>(sq[j] + st * 2);
              w[0] = v.x; w[1] = v.y; w[2] = v.z; w[3] = v.w;
            } else {
              const u32x2 v = *reinterpret_cast<const u32x2*>(sq[j] + st * 2);
              w[0] = v.x; w[1] = v.y; w[2] = 0u; w[3] = 0u;
            }
#pragma unroll
            for (int u = 0; u < UNROLL; ++u) bv[u][j].s = (w[u / 2] >> ((u % 2) * 16 + sh)) & 0xFFu;
          }
        } else {
#pragma unroll
          for (int u = 0; u < UNROLL; ++u)
#pragma unroll
            for (int j = 0; j < NS; ++j) bv[u][j] = load_b(j, st + u);
        }
#pragma unroll
        for (int u = 0; u < UNROLL; ++u)
#pragma unroll
          for (int t = 0; t < MT; ++t) {
            a0[u][t] = *reinterpret_cast<const u32x4*>(ap[t] + (st + u) * 64);
            a1[u][t] = *reinterpret_cast<const u32x4*>(ap[t] + (st + u) * 64 + 8);
          }
#pragma unroll
        for (int u = 0; u < UNROLL; ++u) mfma_step(bv[u], a0[u], a1[u]);
      }
      for (; st < nsteps; ++st) {
        BRaw bv[NS];
        u32x4 a0[MT], a1[MT];
#pragma unroll
        for (int j = 0; j < NS; ++j) bv[j] = load_b(j, st);
#pragma unroll
        for (int t = 0; t < MT; ++t) {
          a0[t] = *reinterpret_cast<const u32x4*>(ap[t] + st * 64);
          a1[t] = *reinterpret_cast<const u32x4*>(ap[t] + st * 64 + 8);
        }
        mfma_step(bv, a0, a1);
      }
    }
    seg_k0 += S.K;
  }

  if (acc_out != nullptr) {                   // the caller reduces and stores
#pragma unroll
    for (int j = 0; j < NS; ++j)
#pragma unroll
      for (int t = 0; t < MT; ++t) acc_out[j * MT + t] = acc[j][t];
    return;
  }
#pragma unroll
  for (int j = 0; j < NS; ++j) {
    const int n = n_first + j * 16 + (lane >> 4) * 4;
    if (n >= P.N) continue;
#pragma unroll
    for (int t = 0; t < MT; ++t) {
      const int m = t * 16 + (lane & 15);
      if (m >= rows) continue;
      f32x4v v = acc[j][t];
      if (partial != nullptr) {
        *reinterpret_cast<f32x4v*>(partial + (int64_t)(out_row0 + m) * P.N + n) = v;
      } else if (epi == EPI_F32) {
        *reinterpret_cast<f32x4v*>(static_cast<float*>(P.C) + (int64_t)(out_row0 + m) * P.ldc + n) = v;
      } else {
        if (epi == EPI_RELU2_BF16) {
          v[0] = relu2(v[0]); v[1] = relu2(v[1]); v[2] = relu2(v[2]); v[3] = relu2(v[3]);
        }
        *reinterpret_cast<u32x2*>(static_cast<uint16_t*>(P.C) + (int64_t)(out_row0 + m) * P.ldc + n) =
            P.residual ? add_residual_bf16x4(v, P.residual + (int64_t)(out_row0 + m) * P.ldr + n)
                       : u32x2{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
      }
    }
  }
}

// MXFP4 experts in 128-deep k pairs (K a multiple of 128, one K segment, 16
// rows). Lane group g = lane / 16 holds k = 32g .. 32g+31 of a pair, so its
// codes are one 16-byte load and the four lane groups of a row read 64
// consecutive bytes: with 64-deep steps a lane's 8 bytes left each row's cache
// line request serving 32 bytes, and the kernel was bound by those requests.
// The lane's k are one scale block (block g of the pair's four), and MFMA q of
// the pair takes its k 32g + 8q .. +7 of the codes and, in the same order, of
// the activations, so the products are unchanged. The scales of UNROLL pairs
// are a row's 4 * UNROLL consecutive bytes, read in one load.
template <int NS, int UNROLL>
__device__ __forceinline__ void skinny_tile_mx4(const SkinnyProblem& P, int n_first, int rows, int row0,
                                                const int32_t* gather, int64_t b_base, int out_row0, int lane,
                                                int epi) {
  static_assert(UNROLL == 4, "scale block of four pairs");
  const KSeg& S = P.seg[0];
  const int g = lane >> 4;
  const int m = min(lane & 15, rows - 1);
  const int64_t arow = gather ? (int64_t)gather[row0 + m] : (int64_t)(row0 + m);
  const uint16_t* ap = S.A + arow * S.lda + 32 * g;
  const uint8_t* cp[NS];
  const uint8_t* sq[NS];
#pragma unroll
  for (int j = 0; j < NS; ++j) {
    const int nr = min(n_first + j * 16 + (lane & 15), P.Nb - 1);
    cp[j] = P.mx_codes + (b_base + (int64_t)nr * S.ldb + 32 * g) / 2;
    sq[j] = P.mx_scales + b_base / 32 + (int64_t)nr * (S.ldb / 32);
  }
  f32x4v acc[NS];
#pragma unroll
  for (int j = 0; j < NS; ++j) acc[j] = f32x4v{0.f, 0.f, 0.f, 0.f};
  const bool sblock = (S.ldb / 32) % (4 * UNROLL) == 0 && (b_base / 32) % (4 * UNROLL) == 0 &&
                      (reinterpret_cast<uintptr_t>(P.mx_scales) & (4 * UNROLL - 1)) == 0;
  auto pair = [&](const u32x4 (&c)[NS], const uint32_t (&sc)[NS], const u32x4 (&a)[4]) {
#pragma unroll
    for (int j = 0; j < NS; ++j)
#pragma unroll
      for (int q = 0; q < 4; ++q)
        acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, mx4_decode8(c[j][q], sc[j])),
                                                         __builtin_bit_cast(bf16x8, a[q]), acc[j], 0, 0, 0);
  };
  const int npairs = S.K / 128;
  int p = 0;
  for (; p + UNROLL <= npairs; p += UNROLL) {
    u32x4 c[UNROLL][NS], a[UNROLL][4];
    uint32_t sc[UNROLL][NS];
#pragma unroll
    for (int u = 0; u < UNROLL; ++u)
#pragma unroll
      for (int j = 0; j < NS; ++j) c[u][j] = *reinterpret_cast<const u32x4*>(cp[j] + (p + u) * 64);
#pragma unroll
    for (int j = 0; j < NS; ++j) {
      if (sblock) {
        const u32x4 w = *reinterpret_cast<const u32x4*>(sq[j] + 4 * p);
#pragma unroll
        for (int u = 0; u < UNROLL; ++u) sc[u][j] = (w[u] >> (8 * g)) & 0xFFu;
      } else {
#pragma unroll
        for (int u = 0; u < UNROLL; ++u) sc[u][j] = sq[j][4 * (p + u) + g];
      }
    }
#pragma unroll
    for (int u = 0; u < UNROLL; ++u)
#pragma unroll
      for (int q = 0; q < 4; ++q) a[u][q] = *reinterpret_cast<const u32x4*>(ap + (p + u) * 128 + 8 * q);
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) pair(c[u], sc[u], a[u]);
  }
  for (; p < npairs; ++p) {
    u32x4 c[NS], a[4];
    uint32_t sc[NS];
#pragma unroll
    for (int j = 0; j < NS; ++j) {
      c[j] = *reinterpret_cast<const u32x4*>(cp[j] + p * 64);
      sc[j] = sq[j][4 * p + g];
    }
#pragma unroll
    for (int q = 0; q < 4; ++q) a[q] = *reinterpret_cast<const u32x4*>(ap + p * 128 + 8 * q);
    pair(c, sc, a);
  }
  // lane l holds row l % 16 and columns 4 * (l / 16) + 0..3 of each slab
  const int mr = lane & 15;
  if (mr >= rows) return;
#pragma unroll
  for (int j = 0; j < NS; ++j) {
    const int n = n_first + j * 16 + (lane >> 4) * 4;
    if (n >= P.N) continue;
    f32x4v v = acc[j];
    if (epi == EPI_RELU2_BF16) {
      v[0] = relu2(v[0]); v[1] = relu2(v[1]); v[2] = relu2(v[2]); v[3] = relu2(v[3]);
    }
    *reinterpret_cast<u32x2*>(static_cast<uint16_t*>(P.C) + (int64_t)(out_row0 + mr) * P.ldc + n) =
        u32x2{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
  }
}

// Dense products of 33..64 rows (a 64-token decode's fc1, shared up and fc2 +
// shared down). With the rows in registers every wave reads all of them for
// its k range: as many bytes of activations as of weights per step, each row a
// cache-line request of its own, and the product ran at 1.7-2.6 TB/s. Here a
// workgroup's four waves take 256 adjacent columns (4 slabs of 16 each) of one
// k split, and a step's activations (64 rows x 64 k, 8 KB) are loaded once
// into LDS (global -> LDS directly, two stages, the tiled GEMM's swizzle) and
// read from there by the four waves; each wave streams its weights straight
// into registers one step ahead, as the other skinny products do. One barrier
// per step. Same k order and MFMA as skinny_tile (lane group g holds k 16g ..
// 16g+15 of a step), so the products are the same.
constexpr int kDense64Cols = 256;             // columns per workgroup
__global__ void __launch_bounds__(256) skinny_dense64_kernel(const SkinnyProblem P) {
  __shared__ u32x4 act[2][64 * 8];            // two stages of 64 rows x 8 chunks of 16 bytes
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int ngroups = (P.N + kDense64Cols - 1) / kDense64Cols;
  const int ks = (int)blockIdx.x % P.ksplit, cg = (int)blockIdx.x / P.ksplit;
  if (cg >= ngroups) return;
  const int n_first = cg * kDense64Cols + wave * 64;
  const bool active = n_first < P.N;          // a wave past the last column still loads and waits
  const int M = P.M;
  int ktot = 0;
  for (int s = 0; s < P.nseg; ++s) ktot += P.seg[s].K;
  const int ksteps = ktot / 64;
  const int k_begin = (int)((int64_t)ksteps * ks / P.ksplit) * 64;
  const int k_end = (int)((int64_t)ksteps * (ks + 1) / P.ksplit) * 64;
  float* partial = P.partial ? P.partial + (int64_t)ks * P.M * P.N : nullptr;
  const int g = lane >> 4, r16 = lane & 15;

  // this thread's two 16-byte chunks of a step's activations: LDS position p,
  // row p / 8, slot p % 8 holding logical chunk swz_slot(row, slot) (rows past
  // M repeat the last row; their results are not stored)
  int drow[2], dchk[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int p = (wave * 2 + i) * 64 + lane;
    drow[i] = min(p / 8, M - 1);
    dchk[i] = swz_slot(p / 8, p % 8);
  }
  f32x4v acc[4][4];
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int t = 0; t < 4; ++t) acc[j][t] = f32x4v{0.f, 0.f, 0.f, 0.f};

  int seg_k0 = 0;
  for (int s = 0; s < P.nseg; ++s) {
    const KSeg& S = P.seg[s];
    const int lo = max(k_begin, seg_k0), hi = min(k_end, seg_k0 + S.K);
    if (lo < hi) {                            // the same for the four waves
      const int nsteps = (hi - lo) / 64;
      const __amdgpu_buffer_rsrc_t ra = make_rsrc(S.A);
      uint32_t ao[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) ao[i] = (uint32_t)((int64_t)drow[i] * S.lda * 2 + dchk[i] * 16);
      auto dma = [&](int st, int stage) {
        const int so = (lo - seg_k0 + st * 64) * 2;
#pragma unroll
        for (int i = 0; i < 2; ++i)
          __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, (lds_void_ptr)&act[stage][(wave * 2 + i) * 64], 16, (int)ao[i],
                                                   so, 0, 0);
      };
      const uint16_t* bp[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int nr = min(n_first + j * 16 + r16, P.Nb - 1);
        bp[j] = S.B + (int64_t)nr * S.ldb + (lo - seg_k0) + 16 * g;
      }
      struct W {
        u32x4 w0[4], w1[4];
      };
      auto wload = [&](int st) {
        W r;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          r.w0[j] = *reinterpret_cast<const u32x4*>(bp[j] + st * 64);
          r.w1[j] = *reinterpret_cast<const u32x4*>(bp[j] + st * 64 + 8);
        }
        return r;
      };
      W cur{}, nxt{};
      dma(0, 0);
      if (active) cur = wload(0);
      MOE_WAIT_VMCNT(0);
      __syncthreads();
      for (int st = 0; st < nsteps; ++st) {
        const int stg = st & 1;
        if (st + 1 < nsteps) {
          if (active) nxt = wload(st + 1);
          dma(st + 1, stg ^ 1);
        }
        u32x4 a0[4], a1[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const int r = t * 16 + r16;
          a0[t] = act[stg][r * 8 + swz_slot(r, 2 * g)];
          a1[t] = act[stg][r * 8 + swz_slot(r, 2 * g + 1)];
        }
        if (active) {
#pragma unroll
          for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int t = 0; t < 4; ++t) {
              acc[j][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, cur.w0[j]),
                                                                  __builtin_bit_cast(bf16x8, a0[t]), acc[j][t], 0, 0, 0);
              acc[j][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, cur.w1[j]),
                                                                  __builtin_bit_cast(bf16x8, a1[t]), acc[j][t], 0, 0, 0);
            }
        }
        // the next step's activations have landed (every wave waited for its
        // own loads) and nobody reads this stage any more
        MOE_WAIT_VMCNT(0);
        __syncthreads();
        cur = nxt;
      }
    }
    seg_k0 += S.K;
  }
  if (!active) return;
  const int epi = P.epi;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int n = n_first + j * 16 + (lane >> 4) * 4;
    if (n >= P.N) continue;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const int m = t * 16 + (lane & 15);
      if (m >= M) continue;
      f32x4v v = acc[j][t];
      if (partial != nullptr) {
        *reinterpret_cast<f32x4v*>(partial + (int64_t)m * P.N + n) = v;
      } else if (epi == EPI_F32) {
        *reinterpret_cast<f32x4v*>(static_cast<float*>(P.C) + (int64_t)m * P.ldc + n) = v;
      } else {
        if (epi == EPI_RELU2_BF16) {
          v[0] = relu2(v[0]); v[1] = relu2(v[1]); v[2] = relu2(v[2]); v[3] = relu2(v[3]);
        }
        *reinterpret_cast<u32x2*>(static_cast<uint16_t*>(P.C) + (int64_t)m * P.ldc + n) =
            P.residual ? add_residual_bf16x4(v, P.residual + (int64_t)m * P.ldr + n)
                       : u32x2{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
      }
    }
  }
}

// One wavefront per (group, column block, k split); 4 waves per workgroup. A
// column block is NSB slabs of 16 columns.
// GROUPED_EPI: -1 for dense products (epilogue from the problem), else the
// fixed epilogue of a grouped expert product (which also names up and down
// apart in profiles).
constexpr int unroll_steps(int mt, int nsb, int bmode) {
  const bool mx = bmode == kSkinnyMx || bmode == kSkinnyMx4;
  const int bytes = bmode == kSkinnyMx ? 16 : bmode == kSkinnyMx4 ? 8 : bmode == kSkinnyF32 ? 64 : 32;
  int u = (mx ? MOE_SKINNY_MX_INFLIGHT : MOE_SKINNY_INFLIGHT) / (nsb * mt * bytes);
  // the activation fragments of the steps in flight take 8 registers each per m-tile
  if (u > 8 / mt) u = 8 / mt;
  return u > 0 ? u : 1;
}

template <int NSB, int GROUPED_EPI, int BMODE = kSkinnyBf16>
__global__ void __launch_bounds__(256) skinny_kernel(const SkinnyProblem P) {
  const int lane = threadIdx.x & 63;
  const int64_t task = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int nblocks = (P.N + 16 * NSB - 1) / (16 * NSB);
  const int64_t per_group = (int64_t)nblocks * P.ksplit;
  const int gi = (int)(task / per_group);
  if (gi >= P.groups) return;
  const int rem = (int)(task - (int64_t)gi * per_group);
  const int blk = rem / P.ksplit, ks = rem % P.ksplit;

  int row0 = 0, rows = P.M;
  int64_t b_base = 0;
  if (P.offsets != nullptr) {            // grouped: the gi-th expert with tokens
    if (gi >= *P.n_groups) return;
    const int g = P.group_list[gi];
    row0 = P.offsets[g];
    rows = P.offsets[g + 1] - row0;
    b_base = (int64_t)g * P.b_estride;
  }
  if (rows <= 0) return;

  int ktot = 0;
  for (int s = 0; s < P.nseg; ++s) ktot += P.seg[s].K;
  const int ksteps = ktot / 64;
  const int k_begin = (int)((int64_t)ksteps * ks / P.ksplit) * 64;
  const int k_end = (int)((int64_t)ksteps * (ks + 1) / P.ksplit) * 64;
  float* partial = P.partial ? P.partial + (int64_t)ks * P.M * P.N : nullptr;
  const int n_first = blk * 16 * NSB;
  const int epi = GROUPED_EPI >= 0 ? GROUPED_EPI : P.epi;

  if constexpr (BMODE == kSkinnyMx || BMODE == kSkinnyMx4) {
    // MX experts: passes of 16 rows (an expert of a decode batch has a few;
    // more rows read its weights again). Keeping only the one-tile variant
    // leaves room for twice the codes in flight per lane at the same occupancy.
    if constexpr (BMODE == kSkinnyMx4) {
      if (GROUPED_EPI >= 0 && P.partial == nullptr && P.residual == nullptr && P.seg[0].K % 128 == 0) {
        for (int r0 = 0; r0 < rows; r0 += 16)
          skinny_tile_mx4<NSB, 4>(P, n_first, min(16, rows - r0), row0 + r0, P.gather, b_base, row0 + r0, lane, epi);
        return;
      }
    }
    for (int r0 = 0; r0 < rows; r0 += 16)
      skinny_tile<1, NSB, unroll_steps(1, NSB, BMODE), BMODE>(P, n_first, min(16, rows - r0), row0 + r0, P.gather,
                                                             b_base, k_begin, k_end, row0 + r0, partial, lane, epi);
    return;
  }
  // up to 64 rows in registers per pass; more rows take further passes
  for (int r0 = 0; r0 < rows; r0 += 64) {
    const int rr = min(64, rows - r0);
    // steps in flight per lane: about 128 bytes of weights
    if (rr <= 16)
      skinny_tile<1, NSB, unroll_steps(1, NSB, BMODE), BMODE>(P, n_first, rr, row0 + r0, P.gather, b_base, k_begin,
                                                             k_end, row0 + r0, partial, lane, epi);
    else if (rr <= 32)
      skinny_tile<2, NSB, unroll_steps(2, NSB, BMODE), BMODE>(P, n_first, rr, row0 + r0, P.gather, b_base, k_begin,
                                                             k_end, row0 + r0, partial, lane, epi);
    else
      skinny_tile<4, NSB, unroll_steps(4, NSB, BMODE), BMODE>(P, n_first, rr, row0 + r0, P.gather, b_base, k_begin,
                                                             k_end, row0 + r0, partial, lane, epi);
  }
}

// Dense products of 1..16 rows with K split inside the workgroup: the KW waves
// of a workgroup take KW consecutive k ranges of one 16-column slab, leave their
// fp32 sums in LDS, and wave 0 adds them in wave order and applies the
// epilogue. The same fixed order on every call, no partials in global memory
// and no reduction launch (the split over workgroups needed a second pass).
// Up to two problems per launch (fc1 and the shared expert's up product read
// the same rows): workgroup b < slabs0 takes slab b of the first.
struct SkinnyPair {
  SkinnyProblem p[2];
  int slabs0;                // slabs of p[0]; the workgroups after them take p[1]
};

template <int KW>
__global__ void __launch_bounds__(64 * KW) skinny_wgk_kernel(const SkinnyPair L) {
  __shared__ f32x4v red[KW][64];
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  int slab = blockIdx.x;
  const int pi = slab >= L.slabs0 ? 1 : 0;
  slab -= pi * L.slabs0;
  const SkinnyProblem& P = L.p[pi];
  const int n_first = slab * 16;
  int ktot = 0;
  for (int s = 0; s < P.nseg; ++s) ktot += P.seg[s].K;
  const int ksteps = ktot / 64;
  const int k_begin = ksteps * w / KW * 64, k_end = ksteps * (w + 1) / KW * 64;
  f32x4v acc;
  skinny_tile<1, 1, unroll_steps(1, 1, kSkinnyBf16), kSkinnyBf16>(P, n_first, P.M, 0, nullptr, 0, k_begin, k_end, 0,
                                                                   nullptr, lane, P.epi, &acc);
  red[w][lane] = acc;
  __syncthreads();
  if (w != 0) return;
  f32x4v v = red[0][lane];
#pragma unroll
  for (int i = 1; i < KW; ++i) v += red[i][lane];
  // lane l holds row l % 16 and columns 4 * (l / 16) + 0..3 of the slab
  const int m = lane & 15, n = n_first + (lane >> 4) * 4;
  if (m >= P.M || n >= P.N) return;
  if (P.epi == EPI_F32) {
    *reinterpret_cast<f32x4v*>(static_cast<float*>(P.C) + (int64_t)m * P.ldc + n) = v;
    return;
  }
  if (P.epi == EPI_RELU2_BF16) {
    v[0] = relu2(v[0]); v[1] = relu2(v[1]); v[2] = relu2(v[2]); v[3] = relu2(v[3]);
  }
  *reinterpret_cast<u32x2*>(static_cast<uint16_t*>(P.C) + (int64_t)m * P.ldc + n) =
      P.residual ? add_residual_bf16x4(v, P.residual + (int64_t)m * P.ldr + n)
                 : u32x2{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
}

constexpr int kWgkWaves = 16;

hipError_t launch_skinny_wgk(const SkinnyProblem& P0, const SkinnyProblem* P1, hipStream_t st) {
  const int s0 = (P0.N + 15) / 16;
  const int s1 = P1 ? (P1->N + 15) / 16 : 0;
  if (s0 + s1 <= 0) return hipSuccess;
  SkinnyPair L;
  L.p[0] = P0;
  L.p[1] = P1 ? *P1 : P0;
  L.slabs0 = s0;
  hipLaunchKernelGGL(skinny_wgk_kernel<kWgkWaves>, dim3(s0 + s1), dim3(64 * kWgkWaves), 0, st, L);
  return hipGetLastError();
}

// out[m, n] = epi(sum_{s < ksplit} partial[s, m, n]), summed in split order.
__global__ void __launch_bounds__(256) skinny_reduce_kernel(const float* __restrict__ partial, int ksplit, int M, int N,
                                                            void* C, int64_t ldc, int epi,
                                                            const uint16_t* __restrict__ residual, int64_t ldr) {
  const int64_t i = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) * 4;
  const int64_t total = (int64_t)M * N;
  if (i >= total) return;
  f32x4v s = *reinterpret_cast<const f32x4v*>(partial + i);
  for (int k = 1; k < ksplit; ++k) s += *reinterpret_cast<const f32x4v*>(partial + (int64_t)k * total + i);
  const int m = (int)(i / N), n = (int)(i % N);
  if (epi == EPI_F32) {
    *reinterpret_cast<f32x4v*>(static_cast<float*>(C) + (int64_t)m * ldc + n) = s;
  } else {
    if (epi == EPI_RELU2_BF16) {
      s[0] = relu2(s[0]); s[1] = relu2(s[1]); s[2] = relu2(s[2]); s[3] = relu2(s[3]);
    }
    *reinterpret_cast<u32x2*>(static_cast<uint16_t*>(C) + (int64_t)m * ldc + n) =
        residual ? add_residual_bf16x4(s, residual + (int64_t)m * ldr + n)
                 : u32x2{pack_bf16x2(s[0], s[1]), pack_bf16x2(s[2], s[3])};
  }
}

// The same for few outputs and many splits (a decode router or fc1: hundreds of
// outputs, tens of splits), where one thread per output would walk its splits
// one dependent load after another: one wave per 4 outputs, lane l summing
// splits l, l + 64, ..., then a fixed butterfly over the wave (the same order
// every call).
__global__ void __launch_bounds__(256) skinny_reduce_wide_kernel(const float* __restrict__ partial, int ksplit, int M,
                                                                 int N, void* C, int64_t ldc, int epi,
                                                                 const uint16_t* __restrict__ residual, int64_t ldr) {
  const int lane = threadIdx.x & 63;
  const int64_t i = ((int64_t)blockIdx.x * 4 + (threadIdx.x >> 6)) * 4;
  const int64_t total = (int64_t)M * N;
  if (i >= total) return;
  f32x4v s = f32x4v{0.f, 0.f, 0.f, 0.f};
  for (int k = lane; k < ksplit; k += 64) s += *reinterpret_cast<const f32x4v*>(partial + (int64_t)k * total + i);
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) {
#pragma unroll
    for (int q = 0; q < 4; ++q) s[q] += __shfl_xor(s[q], m, 64);
  }
  if (lane != 0) return;
  const int m = (int)(i / N), n = (int)(i % N);
  if (epi == EPI_F32) {
    *reinterpret_cast<f32x4v*>(static_cast<float*>(C) + (int64_t)m * ldc + n) = s;
  } else {
    if (epi == EPI_RELU2_BF16) {
      s[0] = relu2(s[0]); s[1] = relu2(s[1]); s[2] = relu2(s[2]); s[3] = relu2(s[3]);
    }
    *reinterpret_cast<u32x2*>(static_cast<uint16_t*>(C) + (int64_t)m * ldc + n) =
        residual ? add_residual_bf16x4(s, residual + (int64_t)m * ldr + n)
                 : u32x2{pack_bf16x2(s[0], s[1]), pack_bf16x2(s[2], s[3])};
  }
}

hipError_t launch_skinny(const SkinnyProblem& P, hipStream_t st, bool reduce) {
  // dense products carry up to 64 rows: 4 slabs per wave load the rows once per
  // four weight fragments; grouped products have a few rows per expert
  const int nsb = skinny_slabs_per_wave(P);
  const int64_t nblocks = (P.N + 16 * nsb - 1) / (16 * nsb);
  const int64_t tasks = (int64_t)P.groups * nblocks * P.ksplit;
  if (tasks <= 0) return hipSuccess;
  const dim3 grid((unsigned)((tasks + 3) / 4)), block(256);
  if (P.offsets == nullptr) {
    if (P.mx_codes != nullptr) return hipErrorInvalidValue;     // MX weights: grouped products only
    if (P.f32_b == nullptr && P.M > 32 && P.M <= 64 && MOE_SKINNY_DENSE64) {
      // 33..64 rows, bf16 weights: the activations of a step shared through LDS
      const int64_t wgs = (int64_t)((P.N + kDense64Cols - 1) / kDense64Cols) * P.ksplit;
      hipLaunchKernelGGL(skinny_dense64_kernel, dim3((unsigned)wgs), dim3(256), 0, st, P);
    } else if (P.f32_b != nullptr) {                                   // fp32 weights: one K segment
      if (P.nseg != 1) return hipErrorInvalidValue;
      if (nsb == 4) hipLaunchKernelGGL((skinny_kernel<4, -1, kSkinnyF32>), grid, block, 0, st, P);
      else hipLaunchKernelGGL((skinny_kernel<1, -1, kSkinnyF32>), grid, block, 0, st, P);
    } else if (nsb == 4) {
      hipLaunchKernelGGL((skinny_kernel<4, -1>), grid, block, 0, st, P);
    } else {
      hipLaunchKernelGGL((skinny_kernel<1, -1>), grid, block, 0, st, P);
    }
  } else {
    if (P.f32_b != nullptr) return hipErrorInvalidValue;        // fp32 weights: dense products only
    if (P.mx_codes != nullptr && P.nseg != 1) return hipErrorInvalidValue;
    const bool relu2 = P.epi == EPI_RELU2_BF16, mx = P.mx_codes != nullptr;
    const bool fp4 = mx && P.mx_fp4;
#define MOE_GROUPED_MX(NS, FMT)                                                                             \
  if (relu2) hipLaunchKernelGGL((skinny_kernel<NS, EPI_RELU2_BF16, FMT>), grid, block, 0, st, P);          \
  else hipLaunchKernelGGL((skinny_kernel<NS, EPI_BF16, FMT>), grid, block, 0, st, P);
    if (nsb == 4 && fp4) {                                      // MX only, see skinny_slabs_per_wave
      MOE_GROUPED_MX(4, kSkinnyMx4)
    } else if (nsb == 4) {
      MOE_GROUPED_MX(4, kSkinnyMx)
    } else if (fp4) {
      MOE_GROUPED_MX(1, kSkinnyMx4)
    } else if (mx) {
      MOE_GROUPED_MX(1, kSkinnyMx)
    } else if (relu2) {
      hipLaunchKernelGGL((skinny_kernel<1, EPI_RELU2_BF16>), grid, block, 0, st, P);
    } else {
      hipLaunchKernelGGL((skinny_kernel<1, EPI_BF16>), grid, block, 0, st, P);
    }
#undef MOE_GROUPED_MX
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || P.partial == nullptr || !reduce) return e;
  const int64_t total = (int64_t)P.M * P.N;
  if (P.ksplit >= 16 && total / 4 <= 4096)
    hipLaunchKernelGGL(skinny_reduce_wide_kernel, dim3((unsigned)((total / 4 + 3) / 4)), dim3(256), 0, st, P.partial,
                       P.ksplit, P.M, P.N, P.C, P.ldc, P.epi, P.residual, P.ldr);
  else
    hipLaunchKernelGGL(skinny_reduce_kernel, dim3((unsigned)((total / 4 + 255) / 256)), dim3(256), 0, st, P.partial,
                       P.ksplit, P.M, P.N, P.C, P.ldc, P.epi, P.residual, P.ldr);
  return hipGetLastError();
}

}  // namespace moe
