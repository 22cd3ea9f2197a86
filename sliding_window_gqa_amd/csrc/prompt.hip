// Prompt rows of windowed GQA attention on gfx950: MFMA tiled online softmax.
//
// Method: TensorFold pull request #1123, "window_attention at head dim 256", section
// "What this changes", Prompt, Window.p32 and promptRows(..., hi) bullets. Each row i sees
// keys [lo_i, last_i]; keys come in tiles at absolute positions; every tile folds into the
// running (m, l, O) of a row with one rescale; P enters P.V as one bf16 or, with p32, as
// bf16(P) followed by bf16(P - bf16(P)). A tile that holds none of a row's keys leaves that
// row's state exactly unchanged (alpha = 1, P = 0), so a row's bits depend only on its own
// key range and the absolute tile grid, never on how the prompt is cut into calls.
//
// gfx950 design (own, not the page's tensor-core layout):
//   * a workgroup holds 4 waves; each wave owns 32 (row, query head) pairs of one key head,
//     so the G query heads of a key head share every K/V tile (GQA folded into the MFMA N
//     dimension, rows x heads);
//   * v_mfma_f32_32x32x16_bf16 computes S^T = K Q^T (keys x pairs) and O^T += V^T P^T
//     (dims x pairs). With the transposed products every lane holds a single pair (lane % 32)
//     in all of S, P and O, so the row max, the rescale and the sum are lane-local plus one
//     exchange between the two lane halves;
//   * K tiles sit in LDS as [key][dim]; V tiles are transposed on their way into LDS
//     ([dim][key]) so both MFMA operands are 16-byte LDS reads;
//   * the K rows of a tile are fed to the first MFMA in a permuted order so that the S^T
//     accumulator registers of a lane are, eight at a time, exactly the B operand (P^T) the
//     P.V MFMA needs for eight consecutive keys: no shuffles between the two products;
//   * the workgroup index is remapped so that each XCD (8 on MI355X, workgroups dealt out
//     round-robin) works through a contiguous range of (key head, row block) tiles, keeping
//     a key head's K/V stream in that XCD's L2.
#include "wa_common.h"

namespace wa {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kPairs = 32 * kWaves;   // (row, head) pairs per workgroup
constexpr int BN = 64;                // keys per tile
constexpr float kLog2e = 1.4426950408889634f;

union Pack8 {
    bf16x8 v;
    uint4 u;
    uint32_t w[4];
};

// M-index i of the S^T tile (0..31) -> key within the 32-key half-tile. Lane half h holds
// M-indices 8a + 4h + b (a, b in 0..3); this order makes its registers 8s..8s+7 the keys
// 16s + 8h + 0..7.
__device__ __forceinline__ int sigma(int i) {
    const int a = i >> 3, h = (i >> 2) & 1, b = i & 3;
    return 16 * (a >> 1) + 8 * h + 4 * (a & 1) + b;
}

__device__ __forceinline__ int wave_min_i(int x) {
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) x = min(x, __shfl_xor(x, m, 64));
    return x;
}
__device__ __forceinline__ int wave_max_i(int x) {
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) x = max(x, __shfl_xor(x, m, 64));
    return x;
}

template <int D, bool P32>
__global__ __launch_bounds__(kThreads) void prompt_kernel(PromptArgs a, int nblk) {
    constexpr int KSTEPS = D / 16;
    constexpr int DBLK = D / 32;
    constexpr int KS = D + 8;      // K tile row stride (elements)
    constexpr int VS = BN + 8;     // V^T tile row stride (elements)
    __shared__ __attribute__((aligned(16))) uint16_t Ks[BN * KS];
    __shared__ __attribute__((aligned(16))) uint16_t VT[D * VS];
    __shared__ int red_i[4][kWaves];

    // XCD-aware remap of the linear workgroup index
    const int total = gridDim.x;
    const int L = blockIdx.x;
    const int xcd = L & 7, idx = L >> 3;
    const int per = total >> 3, extra = total & 7;
    const int logical = (xcd < extra ? xcd * (per + 1) : extra * (per + 1) + (xcd - extra) * per) + idx;
    const int g = logical / nblk;           // key head
    const int blk = logical % nblk;         // block of pairs

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int h = lane >> 5;                // lane half
    const int col = lane & 31;              // pair within the wave
    const int G = a.hq / a.hkv;

    const int pair = blk * kPairs + wave * 32 + col;
    const int row = pair / G;
    const int head = g * G + pair % G;
    const bool valid = row < a.n;

    int lo = 1, last = 0;                   // empty range for padding pairs
    if (valid) {
        const int p = a.p0 + row;
        lo = a.window > 0 ? max(0, p - a.window + 1) : 0;
        last = p;
        if (a.hi) {
            int hv = a.hi[row];
            hv = hv < p ? p : (hv > a.p0 + a.n - 1 ? a.p0 + a.n - 1 : hv);
            last = hv;
        }
    }
    // workgroup key range and the range every valid pair sees
    {
        const int big = 0x7FFFFFFF;
        int v0 = wave_min_i(valid ? lo : big);
        int v1 = wave_max_i(valid ? last : -1);
        int v2 = wave_max_i(valid ? lo : -1);
        int v3 = wave_min_i(valid ? last : big);
        if (lane == 0) { red_i[0][wave] = v0; red_i[1][wave] = v1; red_i[2][wave] = v2; red_i[3][wave] = v3; }
    }
    __syncthreads();
    int kmin = red_i[0][0], kmax = red_i[1][0], lo_all = red_i[2][0], last_all = red_i[3][0];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) {
        kmin = min(kmin, red_i[0][w]); kmax = max(kmax, red_i[1][w]);
        lo_all = max(lo_all, red_i[2][w]); last_all = min(last_all, red_i[3][w]);
    }
    if (kmax < kmin) return;                // no valid pair in this workgroup

    // Q^T operand: this lane's pair, dims 16*ks + 8*h + 0..7
    Pack8 qreg[KSTEPS];
    {
        const uint16_t* qp = a.q + (int64_t)row * a.q_srow + (int64_t)head * a.q_shead + 8 * h;
#pragma unroll
        for (int ks = 0; ks < KSTEPS; ++ks) {
            if (valid) qreg[ks].u = *reinterpret_cast<const uint4*>(qp + 16 * ks);
            else qreg[ks].u = make_uint4(0, 0, 0, 0);
        }
    }

    f32x16 oacc[DBLK];
#pragma unroll
    for (int db = 0; db < DBLK; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[db][r] = 0.f;
    float m_run = -INFINITY, l_run = 0.f;
    const float cexp = a.scale * kLog2e;

    const uint16_t* kg = a.k + (int64_t)g * a.kv_shead;
    const uint16_t* vg = a.v + (int64_t)g * a.kv_shead;
    const int krow = sigma(col);            // K row this lane feeds to the S^T MFMA

    for (int tile = kmin / BN; tile <= kmax / BN; ++tile) {
        const int base = tile * BN;
        __syncthreads();
        // K tile -> LDS [key][dim]; keys outside [kmin, kmax] become zeros
        for (int i = tid; i < BN * D / 8; i += kThreads) {
            const int kk = i / (D / 8), dc = i % (D / 8);
            const int j = base + kk;
            uint4 w = make_uint4(0, 0, 0, 0);
            if (j >= kmin && j <= kmax)
                w = *reinterpret_cast<const uint4*>(kg + (int64_t)(j % a.ring) * a.kv_sslot + dc * 8);
            *reinterpret_cast<uint4*>(&Ks[kk * KS + dc * 8]) = w;
        }
        // V tile -> LDS transposed [dim][key], two keys packed per 32-bit store
        for (int i = tid; i < (BN / 2) * (D / 8); i += kThreads) {
            const int kp = i % (BN / 2), dc = i / (BN / 2);
            const int j = base + 2 * kp;
            uint4 w0 = make_uint4(0, 0, 0, 0), w1 = make_uint4(0, 0, 0, 0);
            if (j >= kmin && j <= kmax)
                w0 = *reinterpret_cast<const uint4*>(vg + (int64_t)(j % a.ring) * a.kv_sslot + dc * 8);
            if (j + 1 >= kmin && j + 1 <= kmax)
                w1 = *reinterpret_cast<const uint4*>(vg + (int64_t)((j + 1) % a.ring) * a.kv_sslot + dc * 8);
            const uint32_t x0[4] = {w0.x, w0.y, w0.z, w0.w};
            const uint32_t x1[4] = {w1.x, w1.y, w1.z, w1.w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const uint32_t lo2 = (x0[e] & 0xFFFFu) | (x1[e] << 16);
                const uint32_t hi2 = (x0[e] >> 16) | (x1[e] & 0xFFFF0000u);
                *reinterpret_cast<uint32_t*>(&VT[(dc * 8 + 2 * e) * VS + 2 * kp]) = lo2;
                *reinterpret_cast<uint32_t*>(&VT[(dc * 8 + 2 * e + 1) * VS + 2 * kp]) = hi2;
            }
        }
        __syncthreads();

        // S^T = K Q^T for two 32-key halves
        f32x16 sacc[2];
#pragma unroll
        for (int mb = 0; mb < 2; ++mb) {
#pragma unroll
            for (int r = 0; r < 16; ++r) sacc[mb][r] = 0.f;
            const uint16_t* kp = &Ks[(32 * mb + krow) * KS + 8 * h];
#pragma unroll
            for (int ks = 0; ks < KSTEPS; ++ks) {
                Pack8 av;
                av.u = *reinterpret_cast<const uint4*>(kp + 16 * ks);
                sacc[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av.v, qreg[ks].v, sacc[mb], 0, 0, 0);
            }
        }

        // online softmax in log2 units: t = s * scale * log2(e)
        const bool full = base >= lo_all && base + BN - 1 <= last_all;
        float tmax = -INFINITY;
#pragma unroll
        for (int mb = 0; mb < 2; ++mb)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                float t = sacc[mb][r] * cexp;
                if (!full) {
                    const int kpos = base + 32 * mb + 16 * (r >> 3) + 8 * h + (r & 7);
                    if (kpos < lo || kpos > last) t = -INFINITY;
                }
                sacc[mb][r] = t;
                tmax = fmaxf(tmax, t);
            }
        tmax = fmaxf(tmax, __shfl_xor(tmax, 32, 64));
        const float m_new = fmaxf(m_run, tmax);
        const float mu = (m_new == -INFINITY) ? 0.f : m_new;
        const float alpha = __builtin_amdgcn_exp2f(m_run - mu);
        float psum = 0.f;
#pragma unroll
        for (int mb = 0; mb < 2; ++mb)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const float p = __builtin_amdgcn_exp2f(sacc[mb][r] - mu);
                sacc[mb][r] = p;
                psum += p;
            }
        l_run = fmaf(alpha, l_run, psum);
        m_run = m_new;
#pragma unroll
        for (int db = 0; db < DBLK; ++db)
#pragma unroll
            for (int r = 0; r < 16; ++r) oacc[db][r] *= alpha;

        // O^T += V^T P^T, four 16-key steps
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            const int mb = s >> 1, r0 = (s & 1) * 8;
            Pack8 phi, plo;
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const float p0 = sacc[mb][r0 + 2 * u], p1 = sacc[mb][r0 + 2 * u + 1];
                phi.w[u] = pack_bf16x2(p0, p1);
                if (P32) {
                    const float h0 = lo_bf16(phi.w[u]), h1 = hi_bf16(phi.w[u]);
                    plo.w[u] = pack_bf16x2(p0 - h0, p1 - h1);
                }
            }
#pragma unroll
            for (int db = 0; db < DBLK; ++db) {
                Pack8 av;
                av.u = *reinterpret_cast<const uint4*>(&VT[(32 * db + col) * VS + 16 * s + 8 * h]);
                oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av.v, phi.v, oacc[db], 0, 0, 0);
                if (P32)
                    oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av.v, plo.v, oacc[db], 0, 0, 0);
            }
        }
    }

    // epilogue: O / l, one rounding to bf16
    const float l_tot = l_run + __shfl_xor(l_run, 32, 64);
    if (valid) {
        uint16_t* op = a.out + (int64_t)row * a.o_srow + (int64_t)head * a.o_shead;
#pragma unroll
        for (int db = 0; db < DBLK; ++db)
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4) {
                const int d0 = 32 * db + 8 * q4 + 4 * h;
                uint2 w;
                w.x = pack_bf16x2(oacc[db][4 * q4 + 0] / l_tot, oacc[db][4 * q4 + 1] / l_tot);
                w.y = pack_bf16x2(oacc[db][4 * q4 + 2] / l_tot, oacc[db][4 * q4 + 3] / l_tot);
                *reinterpret_cast<uint2*>(op + d0) = w;
            }
    }
}

template <int D>
hipError_t launch_d(const PromptArgs& a, hipStream_t s) {
    const int G = a.hq / a.hkv;
    const int nblk = (int)(((int64_t)a.n * G + kPairs - 1) / kPairs);
    dim3 grid(nblk * a.hkv);
    if (a.p32) hipLaunchKernelGGL((prompt_kernel<D, true>), grid, dim3(kThreads), 0, s, a, nblk);
    else hipLaunchKernelGGL((prompt_kernel<D, false>), grid, dim3(kThreads), 0, s, a, nblk);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_prompt(const PromptArgs& a, hipStream_t s) {
    return a.d == 256 ? launch_d<256>(a, s) : launch_d<128>(a, s);
}

}  // namespace wa
