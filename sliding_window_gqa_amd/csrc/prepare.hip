// q/k row preparation and the ring write on gfx950: the step on the input side of the
// windowed attention.
//
// Method: TensorFold pull request #1257 ("tf_qk_rows_l2"), "What this changes", and the
// "Exact Numerical Contract" page, "Preparation". For each head of a row at position pos:
//   WA_PREP_ROPE_L2   r = bf16(rope(x)) with fp32 cos/sin of the fp32 angle
//                     fl32(fl32(pos) * inv_j), inv_j = fl32(theta^(-2j/R)) (inv_j from the host);
//                     n = bf16(r * (1 / sqrt(sum r^2 + eps)));  q = bf16(qs * n) if qs given
//   WA_PREP_RMS_ROPE  n = bf16(x * (1 / sqrt(mean x^2 + eps)));
//                     r = bf16(rope(n)) with bf16(cos), bf16(sin) and fp32 arithmetic
//   WA_PREP_COPY      the row as it is (values go into the cache unchanged)
// RoPE is rotate-half over the first R dims, pairs (j, j + R/2); dims R.. pass unrotated.
// The output row goes either to out[row] or, for the caches, to the ring slot pos mod ring
// of the row's stream.
//
// gfx950 mapping: one workgroup of 256 threads per row. The row's R/2 cos/sin pairs are
// computed once (float64 cos and sin of the fp32 angle, each rounded once to fp32, i.e. a
// correctly rounded cosf/sinf; the inverse frequencies come computed by the host) into LDS
// and shared by all heads; the bf16 roundings are hardware conversions (v_cvt_pk_bf16_f32,
// nearest-even). Two forms, the same arithmetic per value:
//   wide    (16-byte aligned rows and heads, R a multiple of 16) a lane holds 8 consecutive
//           dims of a head (one 16-byte load and store), a head is D/8 lanes, and each wave
//           requests up to 8 head groups (every head of a 112-head row at d = 128) before
//           computing any; the head's sum of squares is a lane tree inside its lanes and the
//           rotation partner is the lane R/16 lanes away (one lane permute per value); loads
//           and stores are non-temporal (each byte is touched once);
//   narrow  (anything else) each wave takes heads h = wave, wave + 4, ... and loads a batch
//           of them (14 at d = 128, 8 at d = 256) before computing any: a lane holds D/64
//           consecutive dims (one 4- or 8-byte load), partners of the rotation come through
//           LDS (one row per batch entry, so the heads' chains interleave), the sum of
//           squares is a VALU-only wave sum.
#include "wa_common.h"

namespace wa {

namespace {

constexpr int kPrepThreads = 256;
// heads a wave loads before using any (14 at d = 128: the long prompt's 28 heads a wave in
// two batches; 8 at d = 256, where the LDS staging row is twice as long)
template <int D> constexpr int kBatchOf = D == 128 ? 14 : 8;

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

// two fp32 -> packed bf16 pair (low half first), round to nearest even (v_cvt_pk_bf16_f32)
__device__ __forceinline__ uint32_t pack_bf16(float x, float y) {
    const f32x2_t v = {x, y};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}

// fp32 -> bf16 -> fp32, round to nearest even
__device__ __forceinline__ float round_bf16(float x) { return __uint_as_float(pack_bf16(x, 0.f) << 16); }

template <int CTRL>
__device__ __forceinline__ float dpp_mov(float x) {
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), CTRL, 0xF, 0xF, true));
}

// Sum over the 64 lanes of a wave, the result in every lane, on the VALU only: DPP quad
// permutes and row mirrors inside 16 lanes, then the 16- and 32-lane swaps.
__device__ __forceinline__ float wave_sum64(float v) {
    v += dpp_mov<0xB1>(v);     // quad_perm [1,0,3,2]
    v += dpp_mov<0x4E>(v);     // quad_perm [2,3,0,1]
    v += dpp_mov<0x141>(v);    // row half-mirror: pairs the two quads of each 8 lanes
    v += dpp_mov<0x140>(v);    // row mirror: pairs the two 8-lane halves of each row
    const auto r16 = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    v = __uint_as_float(r16[0]) + __uint_as_float(r16[1]);
    const auto r32 = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return __uint_as_float(r32[0]) + __uint_as_float(r32[1]);
}

template <int D>
__global__ __launch_bounds__(kPrepThreads) void prepare_kernel(PrepArgs a) {
    constexpr int E = D / 64;              // dims per lane
    __shared__ float cs[2][128];           // cos, sin of pair j < R/2 (R <= 256)
    constexpr int kBatch = kBatchOf<D>;
    __shared__ float xs[kPrepThreads / 64][kBatch][D];
    const int r = blockIdx.x;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    int pos = a.pos_of_row[r];
    pos = pos < 0 ? 0 : pos;
    const int R = a.rope_dims, half = R / 2;
    const uint16_t* xrow = a.x + (int64_t)r * a.x_srow;
    constexpr int W = kPrepThreads / 64;
    // a batch of heads: this wave's heads h0, h0 + W, ... (the last head stands in for heads
    // past the end)
    auto load_batch = [&](int h0, uint32_t (&w)[kBatch][E / 2]) {
#pragma unroll
        for (int b = 0; b < kBatch; ++b) {
            const int h = min(h0 + W * b, a.heads - 1);
            const uint16_t* xp = xrow + (int64_t)h * a.x_shead + E * lane;
            if constexpr (E == 4) {
                const uint2 u = *reinterpret_cast<const uint2*>(xp);
                w[b][0] = u.x; w[b][1] = u.y;
            } else {
                w[b][0] = *reinterpret_cast<const uint32_t*>(xp);
            }
        }
    };
    // the first batch's loads are in flight while the row's coefficients are computed
    uint32_t w[kBatch][E / 2];
    load_batch(wave, w);
    if (a.mode != kPrepCopy) {
        for (int j = tid; j < half; j += kPrepThreads) {
            const float ang = (float)pos * a.inv[j];
            double sn, cn;
            sincos((double)ang, &sn, &cn);
            cs[0][j] = (float)cn;
            cs[1][j] = (float)sn;
        }
    }
    __syncthreads();

    uint16_t* orow;
    if (a.ring > 0) {
        int t = a.stream_of_row[r];
        t = t < 0 ? 0 : (t >= a.streams ? a.streams - 1 : t);
        orow = a.out + (int64_t)t * a.o_sstream + (int64_t)(pos % a.ring) * a.o_sslot;
    } else {
        orow = a.out + (int64_t)r * a.o_sslot;
    }
    // this lane's rotation, fixed for the row: dim i = E lane + e pairs with dim pi[e];
    // y = v c + partner s' with s' = -s below R/2 and +s above (bf16 coefficients in the RMS
    // recipe); dims past R keep c = 1, s' = 0
    float cf[E], sf[E];
    int pi[E];
#pragma unroll
    for (int e = 0; e < E; ++e) {
        const int i = E * lane + e;
        cf[e] = 1.f; sf[e] = 0.f; pi[e] = i;
        if (i < R) {
            const int j = i < half ? i : i - half;
            float c = cs[0][j], sn = cs[1][j];
            if (a.mode == kPrepRmsRope) {
                c = bf16_to_f32(f32_to_bf16_rne(c));
                sn = bf16_to_f32(f32_to_bf16_rne(sn));
            }
            cf[e] = c;
            sf[e] = i < half ? -sn : sn;
            pi[e] = i < half ? i + half : i - half;
        }
    }
    // the q scale of this lane's dims (L2 recipe), loaded once
    float qsr[E];
    const bool scaled = a.qs != nullptr;
#pragma unroll
    for (int e = 0; e < E; ++e) qsr[e] = scaled ? a.qs[E * lane + e] : 1.f;
    // rotate-half of the values staged in xw, for element e (the product with -s or +s is
    // exact in sign, so fma(v, c, p * s') is v c -/+ p s with the same two roundings)
    auto rot = [&](const float* xw, float v, int e) {
        if (E * lane + e >= R) return v;
        return fmaf(v, cf[e], xw[pi[e]] * sf[e]);
    };

    // heads in batches of kBatch per wave: the batch's loads are all issued before the
    // first one is used, so a row's memory traffic is in flight together
    for (int h0 = wave; h0 < a.heads; h0 += W * kBatch) {
        if (h0 != wave) load_batch(h0, w);
#pragma unroll
        for (int b = 0; b < kBatch; ++b) {
            const int h = h0 + W * b;
            if (h >= a.heads) break;
            uint16_t* op = orow + (int64_t)h * a.o_shead + E * lane;
            if (a.mode == kPrepCopy) {
                if constexpr (E == 4) *reinterpret_cast<uint2*>(op) = make_uint2(w[b][0], w[b][1]);
                else *reinterpret_cast<uint32_t*>(op) = w[b][0];
                continue;
            }
            float v[E];
#pragma unroll
            for (int e = 0; e < E / 2; ++e) {
                v[2 * e] = lo_bf16(w[b][e]);
                v[2 * e + 1] = hi_bf16(w[b][e]);
            }
            float f[E];                       // the outputs before their bf16 rounding
            float* xw = xs[wave][b];          // one staging row per batch entry: the heads'
                                              // chains can interleave
            if (a.mode == kPrepRopeL2) {
                // r = bf16(rope(x))
#pragma unroll
                for (int e = 0; e < E; ++e) xw[E * lane + e] = v[e];
                __builtin_amdgcn_wave_barrier();
                float rr[E], ss = 0.f;
#pragma unroll
                for (int e = 0; e < E; ++e) {
                    rr[e] = round_bf16(rot(xw, v[e], e));
                    ss = fmaf(rr[e], rr[e], ss);
                }
                __builtin_amdgcn_wave_barrier();
                // n = bf16(r / sqrt(sum r^2 + eps)), q = bf16(qs * n)
                const float inv = 1.0f / sqrtf(wave_sum64(ss) + a.eps);
#pragma unroll
                for (int e = 0; e < E; ++e) {
                    f[e] = rr[e] * inv;
                    if (scaled) f[e] = qsr[e] * round_bf16(f[e]);
                }
            } else {
                // n = bf16(x / sqrt(mean x^2 + eps)), then r = bf16(rope(n)), bf16 coefficients
                float ss = 0.f;
#pragma unroll
                for (int e = 0; e < E; ++e) ss = fmaf(v[e], v[e], ss);
                const float inv = 1.0f / sqrtf(wave_sum64(ss) * (1.0f / D) + a.eps);
                float n[E];
#pragma unroll
                for (int e = 0; e < E; ++e) {
                    n[e] = round_bf16(v[e] * inv);
                    xw[E * lane + e] = n[e];
                }
                __builtin_amdgcn_wave_barrier();
#pragma unroll
                for (int e = 0; e < E; ++e) f[e] = rot(xw, n[e], e);
                __builtin_amdgcn_wave_barrier();
            }
            if constexpr (E == 4) *reinterpret_cast<uint2*>(op) = make_uint2(pack_bf16(f[0], f[1]), pack_bf16(f[2], f[3]));
            else *reinterpret_cast<uint32_t*>(op) = pack_bf16(f[0], f[1]);
        }
    }
}

// The same preparation with 8 dims a lane (16-byte loads and stores): a head is D/8 lanes (4
// heads a wave instruction at d = 128, 2 at d = 256), and a wave requests up to kWideBatch
// such head groups before computing any, which at d = 128 is every head of a 112-head row.
// Sums of squares are lane-tree sums inside the head's lanes; the rotation partner of a lane's
// 8 dims is the lane R/16 lanes away (R a multiple of 16), fetched with one lane permute per
// value. The arithmetic per value is the 2-dims-a-lane kernel's; only the summation order of
// the head's sum of squares differs. Needs 16-byte aligned rows and heads.
constexpr int kWideBatch = 8;
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

template <int D>
__global__ __launch_bounds__(kPrepThreads) void prepare_wide_kernel(PrepArgs a) {
    constexpr int LPH = D / 8;             // lanes a head
    constexpr int HPI = 64 / LPH;          // heads a wave instruction
    constexpr int W = kPrepThreads / 64;
    __shared__ float cs[2][128];           // cos, sin of pair j < R/2 (R <= 256)
    const int r = blockIdx.x;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int lh = lane % LPH, hsub = lane / LPH;
    int pos = a.pos_of_row[r];
    pos = pos < 0 ? 0 : pos;
    const int R = a.rope_dims, half = R / 2;
    const uint16_t* xrow = a.x + (int64_t)r * a.x_srow;
    const int ngroups = (a.heads + HPI - 1) / HPI;
    auto head_of = [&](int grp) { return grp * HPI + hsub; };
    auto load_batch = [&](int g0, uint4 (&w)[kWideBatch]) {
#pragma unroll
        for (int b = 0; b < kWideBatch; ++b) {
            const int h = min(head_of(g0 + W * b), a.heads - 1);
            const u32x4 t = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(xrow + (int64_t)h * a.x_shead + 8 * lh));
            w[b] = make_uint4(t.x, t.y, t.z, t.w);
        }
    };
    // the first batch's loads are in flight while the row's coefficients are computed
    uint4 w[kWideBatch];
    load_batch(wave, w);
    if (a.mode != kPrepCopy) {
        for (int j = tid; j < half; j += kPrepThreads) {
            const float ang = (float)pos * a.inv[j];
            double sn, cn;
            sincos((double)ang, &sn, &cn);
            cs[0][j] = (float)cn;
            cs[1][j] = (float)sn;
        }
    }
    __syncthreads();

    uint16_t* orow;
    if (a.ring > 0) {
        int t = a.stream_of_row[r];
        t = t < 0 ? 0 : (t >= a.streams ? a.streams - 1 : t);
        orow = a.out + (int64_t)t * a.o_sstream + (int64_t)(pos % a.ring) * a.o_sslot;
    } else {
        orow = a.out + (int64_t)r * a.o_sslot;
    }
    // this lane's rotation, fixed for the row: its dims 8 lh .. + 7 all lie below R/2, in
    // [R/2, R) or past R; y = v c + partner s' with s' = -s below R/2 and +s above (bf16
    // coefficients in the RMS recipe); the partner lane is R/16 lanes up or down
    const int d0 = 8 * lh;
    const bool rotd = d0 < R;
    const int plane = d0 < half ? lane + half / 8 : (rotd ? lane - half / 8 : lane);
    float cf[8], sf[8], qsr[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        cf[e] = 1.f; sf[e] = 0.f;
        if (rotd) {
            const int i = d0 + e;
            const int j = i < half ? i : i - half;
            float c = cs[0][j], sn = cs[1][j];
            if (a.mode == kPrepRmsRope) {
                c = bf16_to_f32(f32_to_bf16_rne(c));
                sn = bf16_to_f32(f32_to_bf16_rne(sn));
            }
            cf[e] = c;
            sf[e] = i < half ? -sn : sn;
        }
        qsr[e] = a.qs != nullptr ? a.qs[d0 + e] : 1.f;
    }
    const bool scaled = a.qs != nullptr;
    // sum over the head's LPH lanes (lane-tree inside 16-lane rows, then the 32-lane pair of
    // rows at d = 256), the result in every lane of the head
    auto head_sum = [&](float v) {
        v += dpp_mov<0xB1>(v);     // quad_perm [1,0,3,2]
        v += dpp_mov<0x4E>(v);     // quad_perm [2,3,0,1]
        v += dpp_mov<0x141>(v);    // row half-mirror
        v += dpp_mov<0x140>(v);    // row mirror
        if constexpr (LPH == 32) {
            const auto r16 = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
            v = __uint_as_float(r16[0]) + __uint_as_float(r16[1]);
        }
        return v;
    };
    auto partner = [&](float v) { return __int_as_float(__builtin_amdgcn_ds_bpermute(4 * plane, __float_as_int(v))); };

    for (int g0 = wave; g0 < ngroups; g0 += W * kWideBatch) {
        if (g0 != wave) load_batch(g0, w);
#pragma unroll
        for (int b = 0; b < kWideBatch; ++b) {
            const int grp = g0 + W * b;
            if (grp >= ngroups) break;
            const int h = head_of(grp);
            uint16_t* op = orow + (int64_t)min(h, a.heads - 1) * a.o_shead + d0;
            uint4 res;
            if (a.mode == kPrepCopy) {
                res = w[b];
            } else {
                const uint32_t u[4] = {w[b].x, w[b].y, w[b].z, w[b].w};
                float v[8], f[8];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    v[2 * e] = lo_bf16(u[e]);
                    v[2 * e + 1] = hi_bf16(u[e]);
                }
                if (a.mode == kPrepRopeL2) {
                    // r = bf16(rope(x)); n = bf16(r / sqrt(sum r^2 + eps)); q = bf16(qs * n)
                    float rr[8], ss = 0.f;
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        const float pv = partner(v[e]);
                        rr[e] = round_bf16(rotd ? fmaf(v[e], cf[e], pv * sf[e]) : v[e]);
                        ss = fmaf(rr[e], rr[e], ss);
                    }
                    const float inv = 1.0f / sqrtf(head_sum(ss) + a.eps);
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        f[e] = rr[e] * inv;
                        if (scaled) f[e] = qsr[e] * round_bf16(f[e]);
                    }
                } else {
                    // n = bf16(x / sqrt(mean x^2 + eps)), then r = bf16(rope(n)), bf16
                    // coefficients
                    float ss = 0.f;
#pragma unroll
                    for (int e = 0; e < 8; ++e) ss = fmaf(v[e], v[e], ss);
                    const float inv = 1.0f / sqrtf(head_sum(ss) * (1.0f / D) + a.eps);
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        const float n = round_bf16(v[e] * inv);
                        const float pn = partner(n);
                        f[e] = rotd ? fmaf(n, cf[e], pn * sf[e]) : n;
                    }
                }
                res = make_uint4(pack_bf16(f[0], f[1]), pack_bf16(f[2], f[3]),
                                 pack_bf16(f[4], f[5]), pack_bf16(f[6], f[7]));
            }
            if (h < a.heads) {
                const u32x4 t = {res.x, res.y, res.z, res.w};
                __builtin_nontemporal_store(t, reinterpret_cast<u32x4*>(op));
            }
        }
    }
}

}  // namespace

hipError_t launch_prepare(const PrepArgs& a, hipStream_t s) {
    dim3 grid((unsigned)a.rows);
    // 8 dims a lane where rows and heads are 16-byte aligned and the rotation's half-width is
    // a whole number of lanes; else 2 (d = 128) or 4 (d = 256) dims a lane
    const bool wide = (((uintptr_t)a.x | (uintptr_t)a.out) & 15) == 0 &&
                      ((a.x_srow | a.x_shead | a.o_sstream | a.o_sslot | a.o_shead) & 7) == 0 &&
                      (a.mode == kPrepCopy || a.rope_dims % 16 == 0);
    if (wide) {
        if (a.d == 256) hipLaunchKernelGGL((prepare_wide_kernel<256>), grid, dim3(kPrepThreads), 0, s, a);
        else hipLaunchKernelGGL((prepare_wide_kernel<128>), grid, dim3(kPrepThreads), 0, s, a);
        return hipGetLastError();
    }
    if (a.d == 256) hipLaunchKernelGGL((prepare_kernel<256>), grid, dim3(kPrepThreads), 0, s, a);
    else hipLaunchKernelGGL((prepare_kernel<128>), grid, dim3(kPrepThreads), 0, s, a);
    return hipGetLastError();
}

}  // namespace wa
