// Shared device helpers and the launcher declarations for the wa kernels (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

// Planted mistakes for the GPU control tests, compiled only into separate control builds
// (-DWA_CONTROL=k; the library itself is built with 0). After the planted controls of
// TensorFold pull request #1123 ("Receipt", kernel-contract bullet):
//   1 decode window one key early        2 prompt window one key early
//   3 decode merge without exp(m_c - M)  4 decode merge rounding toward zero
//   5 prompt rows ignoring hi             6 prompt P as one bf16 under p32
#ifndef WA_CONTROL
#define WA_CONTROL 0
#endif

namespace wa {

constexpr int kChunk = 256;      // decode chunk: keys at absolute positions [256c, 256c + 255]

// bf16 bits -> fp32 (exact widening).
__device__ __forceinline__ float bf16_to_f32(uint32_t b) {
    return __uint_as_float(b << 16);
}
// low / high bf16 of a packed pair -> fp32
__device__ __forceinline__ float lo_bf16(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float hi_bf16(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// fp32 -> bf16 bits, round to nearest even; NaN stays NaN, overflow goes to inf, an
// underflow to zero keeps its sign.
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7FFFFFFFu) > 0x7F800000u) return ((u >> 16) & 0x8000u) | 0x7FC0u;
    u += 0x7FFFu + ((u >> 16) & 1u);
    return u >> 16;
}

__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
    return f32_to_bf16_rne(a) | (f32_to_bf16_rne(b) << 16);
}

// Lane exchange across the whole wave (ds_bpermute).
__device__ __forceinline__ float xor_shfl(float x, int mask) {
    return __shfl_xor(x, mask, 64);
}

struct DecodeArgs {
    const uint16_t* q; int64_t q_srow, q_shead;
    const uint16_t* k; const uint16_t* v;
    int64_t kv_sstream, kv_sslot, kv_shead; int32_t streams;
    const int32_t* stream_of_row; const int32_t* pos_of_row; int32_t max_pos;
    int32_t rows, hq, hkv, d;
    int32_t window, ring; float scale;
    int32_t C;                    // chunk capacity of the partial arrays
    float* m; float* l; float* o; // partials
    int32_t rerun;                // 1: re-run non-finite (row, head)s in float64 after the merge
    uint16_t* out; int64_t o_srow, o_shead;
};

// x mod d for a 32-bit unsigned x and 1 <= d < 2^32, from M = floor((2^64 - 1) / d) + 1
// computed once: the high 64 bits of (M x mod 2^64) times d (direct remainder: Lemire, Kaser
// and Kurz, "Faster remainder by direct computation", 2019, exact for every such x and d). A
// division by a value only known at run time costs a long chain of VALU instructions.
inline uint64_t mod_magic(uint32_t d) { return ~0ull / d + 1; }
__device__ __forceinline__ int mod_by_magic(int x, uint64_t M, int d) {
    return (int)__umul64hi(M * (uint32_t)x, (uint64_t)(uint32_t)d);
}

struct PromptArgs {
    const uint16_t* q; int64_t q_srow, q_shead;
    const uint16_t* k; const uint16_t* v; int64_t kv_sslot, kv_shead;
    int32_t p0, n, hq, hkv, d;
    int32_t window, ring; float scale;
    uint64_t ring_magic;          // mod_magic(ring): ring slots of key positions by ring_slot
    int32_t p_parts;              // bf16 parts carrying P into P.V: 1, 2 (p32) or 3
    const int32_t* hi;
    uint16_t* out; int64_t o_srow, o_shead;
    // key-chunk split (windowed prompts): nchunk = key chunks per workgroup grid slot
    // (1 = no split), Cp = chunk capacity per (row, head) of the fp32 partials, chunk_keys =
    // keys per chunk at absolute positions (set by the launcher for the kernel it picks)
    int32_t nchunk, Cp, chunk_keys;
    float* pm; float* pl; float* po;
    // block-sparse prompts: row i sees only the keys of its range whose 64-key block b has
    // bit b % 32 of word b / 32 set in bm[i * bm_srow ..] (words past bm_words: not
    // selected); bm == nullptr: every key of the range
    const uint32_t* bm; int64_t bm_srow; int32_t bm_words;
};

// ring slot of key position x >= 0 of a prompt
__device__ __forceinline__ int ring_slot(const PromptArgs& a, int x) { return mod_by_magic(x, a.ring_magic, a.ring); }


constexpr int kSparseBlock = 64;   // keys per selectable block (= the prompt kernel's key tile)

// is block b selected in a row's mask?
__device__ __forceinline__ bool block_selected(const uint32_t* row_mask, int words, int b) {
    const int w = b >> 5;
    return w < words && ((row_mask[w] >> (b & 31)) & 1u) != 0;
}

// prompt split: keys [384c, 384c + 383], absolute (six 64-key tiles: a 1024-key window over a
// 512-row chunk then fills the GPU in one round of workgroups)
constexpr int kPromptChunk = 384;
// block-sparse prompts at d = 256: 4096-key segments at absolute positions (64 blocks, two mask
// words), one workgroup a (row group, key head, segment)
constexpr int kSparseSeg = 4096;
inline int sparse_segments(int window, int p0, int n) {
    return window > 0 ? (window - 1 + n) / kSparseSeg + 2 : (p0 + n - 1) / kSparseSeg + 1;
}

// (row, query head) pairs per workgroup of the prompt kernel (4 waves of 32)
constexpr int kPromptPairs = 128;

// q/k row preparation (modes as in wa.h)
constexpr int kPrepCopy = 0, kPrepRopeL2 = 1, kPrepRmsRope = 2;
struct PrepArgs {
    int32_t mode, rope_dims; float theta, eps;
    float inv[128];               // fl32(theta^(-2j / rope_dims)), j < rope_dims / 2 (host, float64 pow)
    const uint16_t* x; int64_t x_srow, x_shead;
    const int32_t* pos_of_row; const float* qs;
    int32_t rows, heads, d;
    const int32_t* stream_of_row; int32_t streams, ring;
    uint16_t* out; int64_t o_sstream, o_sslot, o_shead;
};

// Chunk capacities of the windowed-prompt split (both are bounds, independent of the data):
// chunks a workgroup's key range can touch, and chunks one row's key range can touch
// (a row's last key is at most p0 + n - 1, so its range spans at most window - 1 + n keys).
inline int prompt_wg_chunks(int window, int n) { return (window - 1 + n) / kPromptChunk + 2; }
inline int prompt_pair_chunks(int window, int n) { return (window - 1 + n) / kPromptChunk + 2; }
// Sparse prompts are always split; without a window a row's range starts at key 0, so its
// chunks, and a workgroup's, are those of keys 0 .. p0 + n - 1.
inline int sparse_chunks(int window, int p0, int n) {
    return window > 0 ? prompt_pair_chunks(window, n) : (p0 + n - 1) / kPromptChunk + 1;
}

// Launchers: return hipSuccess or the launch error.
hipError_t launch_decode_part(const DecodeArgs& a, hipStream_t s);
// chunk partials + merge, or whole rows in one kernel for large batches (same bits)
hipError_t launch_decode(const DecodeArgs& a, hipStream_t s);
// the decode kernels address a key head's ring with 32-bit offsets: its byte span must be < 2^31
bool decode_extent_ok(int64_t ring, int64_t kv_sslot, int d);
hipError_t launch_merge(const DecodeArgs& a, hipStream_t s);
hipError_t launch_prompt(const PromptArgs& a, hipStream_t s);
hipError_t launch_prepare(const PrepArgs& a, hipStream_t s);

}  // namespace wa
