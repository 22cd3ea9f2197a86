// C ABI of the wa library: argument checks, workspace sizing and kernel dispatch.
// The operation and the conventions are documented in include/wa.h.
#include <cmath>
#include <mutex>

#include "wa_common.h"
#include "../../include/wa.h"

namespace {

bool head_shape_ok(int32_t hq, int32_t hkv, int32_t d) {
    if (d != 128 && d != 256) return false;
    if (hq <= 0 || hkv <= 0 || hq % hkv != 0) return false;
    return hq / hkv <= 16;
}

bool window_ok(const wa_window_t* w) {
    return w && w->window >= 0 && w->ring > 0 && w->scale == w->scale;
}

// The prompt kernel addresses one 64-key tile of K or V with 32-bit byte offsets from the
// tile's first slot: 63 slot strides plus one row must stay below 2^31 bytes.
bool prompt_extent_ok(int64_t kv_sslot, int d) {
    return 63 * kv_sslot * 2 + 2 * (int64_t)d < 0x7FFFFFFF;
}

int chunk_capacity(const wa_window_t* w, int32_t max_pos) {
    if (!window_ok(w) || max_pos < 0) return 0;
    if (w->window > 0) return (w->window - 1 + wa::kChunk - 1) / wa::kChunk + 1;
    return max_pos / wa::kChunk + 1;
}

}  // namespace

extern "C" {

int32_t wa_decode_chunks(const wa_window_t* w, int32_t max_pos) {
    return chunk_capacity(w, max_pos);
}

size_t wa_decode_workspace(int32_t rows, int32_t hq, int32_t d, const wa_window_t* w,
                           int32_t max_pos) {
    const int C = chunk_capacity(w, max_pos);
    if (C <= 0 || rows <= 0 || hq <= 0 || (d != 128 && d != 256)) return 0;
    const size_t cells = (size_t)rows * (size_t)hq * (size_t)C;
    // m and l take an even number of floats each, so that o starts 16-byte aligned
    const size_t cells2 = (cells + 1) & ~(size_t)1;
    return (2 * cells2 + cells * (size_t)d) * sizeof(float);
}

}  // extern "C"

namespace {

// wa_decode's checks and launch; ws is the caller's workspace or this device's scratch
int decode_call(const wa_window_t* w,
                const uint16_t* q, int64_t q_srow, int64_t q_shead,
                const uint16_t* k, const uint16_t* v,
                int64_t kv_sstream, int64_t kv_sslot, int64_t kv_shead, int32_t streams,
                const int32_t* stream_of_row, const int32_t* pos_of_row, int32_t max_pos,
                int32_t rows, int32_t hq, int32_t hkv, int32_t d,
                void* ws, size_t ws_bytes,
                uint16_t* out, int64_t o_srow, int64_t o_shead, void* stream) {
    if (!w || !q || !k || !v || !stream_of_row || !pos_of_row || !out) return WA_EARG;
    if (rows <= 0 || streams <= 0 || max_pos < 0) return WA_EARG;
    if (q_srow < 0 || q_shead < 0 || kv_sstream < 0 || kv_sslot < 0 || kv_shead < 0 ||
        o_srow < 0 || o_shead < 0)
        return WA_EARG;
    if (!head_shape_ok(hq, hkv, d)) return WA_EUNSUPPORTED;
    if (!window_ok(w)) return WA_EARG;
    if (w->window > w->ring) return WA_ERANGE;
    if (w->window == 0 && max_pos >= w->ring) return WA_ERANGE;
    if (!wa::decode_extent_ok(w->ring, kv_sslot, d)) return WA_ERANGE;
    // 16-byte vector loads of q and K/V rows
    if (((uintptr_t)q | (uintptr_t)k | (uintptr_t)v) & 15) return WA_EARG;
    if ((q_srow | q_shead | kv_sstream | kv_sslot | kv_shead) & 7) return WA_EARG;
    const size_t need = wa_decode_workspace(rows, hq, d, w, max_pos);
    if (!ws || ws_bytes < need || need == 0 || ((uintptr_t)ws & 15)) return WA_EWORKSPACE;

    wa::DecodeArgs a{};
    a.q = q; a.q_srow = q_srow; a.q_shead = q_shead;
    a.k = k; a.v = v; a.kv_sstream = kv_sstream; a.kv_sslot = kv_sslot; a.kv_shead = kv_shead;
    a.streams = streams; a.stream_of_row = stream_of_row; a.pos_of_row = pos_of_row;
    a.max_pos = max_pos; a.rows = rows; a.hq = hq; a.hkv = hkv; a.d = d;
    a.window = w->window; a.ring = w->ring; a.scale = w->scale;
    a.C = chunk_capacity(w, max_pos);
    const size_t cells2 = ((size_t)rows * hq * a.C + 1) & ~(size_t)1;
    a.m = static_cast<float*>(ws);
    a.l = a.m + cells2;
    a.o = a.l + cells2;
    a.out = out; a.o_srow = o_srow; a.o_shead = o_shead;
    a.rerun = 1;
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (wa::launch_decode(a, s) != hipSuccess) return WA_EHIP;
    return WA_OK;
}

// Scratch of wa_decode_noalloc: a static device array (each GPU the library runs on holds its
// own copy, for the life of the process). Host code never passes the array's name to a
// kernel (on the host it is only a handle); it passes the device address that
// hipGetSymbolAddress gives, taken once per device with that device current.
__device__ __align__(256) unsigned char scratch[WA_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex scratch_mu;
void* scratch_dev[kMaxDevices];

// this device's scratch address, or nullptr if the device or the symbol query fails
void* scratch_ptr() {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
    std::lock_guard<std::mutex> lock(scratch_mu);
    if (!scratch_dev[dev]) {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess) return nullptr;
        scratch_dev[dev] = p;
    }
    return scratch_dev[dev];
}

}  // namespace

extern "C" {

int wa_decode(const wa_window_t* w,
              const uint16_t* q, int64_t q_srow, int64_t q_shead,
              const uint16_t* k, const uint16_t* v,
              int64_t kv_sstream, int64_t kv_sslot, int64_t kv_shead, int32_t streams,
              const int32_t* stream_of_row, const int32_t* pos_of_row, int32_t max_pos,
              int32_t rows, int32_t hq, int32_t hkv, int32_t d,
              void* ws, size_t ws_bytes,
              uint16_t* out, int64_t o_srow, int64_t o_shead, void* stream) {
    return decode_call(w, q, q_srow, q_shead, k, v, kv_sstream, kv_sslot, kv_shead, streams,
                       stream_of_row, pos_of_row, max_pos, rows, hq, hkv, d, ws, ws_bytes,
                       out, o_srow, o_shead, stream);
}

int wa_decode_noalloc(const wa_window_t* w,
                      const uint16_t* q, int64_t q_srow, int64_t q_shead,
                      const uint16_t* k, const uint16_t* v,
                      int64_t kv_sstream, int64_t kv_sslot, int64_t kv_shead, int32_t streams,
                      const int32_t* stream_of_row, const int32_t* pos_of_row, int32_t max_pos,
                      int32_t rows, int32_t hq, int32_t hkv, int32_t d,
                      uint16_t* out, int64_t o_srow, int64_t o_shead, void* stream) {
    const size_t need = wa_decode_workspace(rows, hq, d, w, max_pos);
    if (need > WA_NOALLOC_SCRATCH_BYTES) return WA_ESCRATCH;
    void* ws = need ? scratch_ptr() : nullptr;
    if (need && !ws) return WA_EHIP;
    // every partial the merge reads is written by the chunk kernel of the same call first,
    // so the scratch needs no clearing between calls
    return decode_call(w, q, q_srow, q_shead, k, v, kv_sstream, kv_sslot, kv_shead, streams,
                       stream_of_row, pos_of_row, max_pos, rows, hq, hkv, d, ws,
                       WA_NOALLOC_SCRATCH_BYTES, out, o_srow, o_shead, stream);
}

int wa_merge(const wa_window_t* w, const float* m, const float* l, const float* o,
             const int32_t* pos_of_row, int32_t rows, int32_t hq, int32_t C, int32_t d,
             uint16_t* out, int64_t o_srow, int64_t o_shead, void* stream) {
    if (!w || !m || !l || !o || !pos_of_row || !out) return WA_EARG;
    if (rows <= 0 || hq <= 0 || C <= 0 || o_srow < 0 || o_shead < 0) return WA_EARG;
    if (d != 128 && d != 256) return WA_EUNSUPPORTED;
    if (!window_ok(w)) return WA_EARG;
    if ((uintptr_t)o & 15) return WA_EARG;   // vector loads of the o partials
    wa::DecodeArgs a{};
    a.m = const_cast<float*>(m); a.l = const_cast<float*>(l); a.o = const_cast<float*>(o);
    a.pos_of_row = pos_of_row; a.rows = rows; a.hq = hq; a.hkv = hq; a.d = d; a.C = C;
    a.window = w->window; a.ring = w->ring; a.scale = w->scale;
    a.max_pos = 0x7FFFFFFF;
    a.out = out; a.o_srow = o_srow; a.o_shead = o_shead;
    a.rerun = 0;   // no q/K/V here: partials made elsewhere are merged as they are
    if (wa::launch_merge(a, static_cast<hipStream_t>(stream)) != hipSuccess) return WA_EHIP;
    return WA_OK;
}

size_t wa_prompt_workspace(const wa_window_t* w, int32_t n, int32_t hq, int32_t d) {
    if (!window_ok(w) || n <= 0 || hq <= 0 || (d != 128 && d != 256)) return 0;
    if (w->window == 0) return 0;
    const size_t cells = (size_t)n * (size_t)hq * (size_t)wa::prompt_pair_chunks(w->window, n);
    return cells * sizeof(float) * (2 + (size_t)d) + 16;   // + alignment slack of the O block
}

int wa_prompt(const wa_window_t* w,
              const uint16_t* q, int64_t q_srow, int64_t q_shead,
              const uint16_t* k, const uint16_t* v, int64_t kv_sslot, int64_t kv_shead,
              int32_t p0, int32_t n, int32_t hq, int32_t hkv, int32_t d,
              const int32_t* hi, void* ws, size_t ws_bytes,
              uint16_t* out, int64_t o_srow, int64_t o_shead, void* stream) {
    if (!w || !q || !k || !v || !out) return WA_EARG;
    if (n <= 0 || p0 < 0) return WA_EARG;
    if (q_srow < 0 || q_shead < 0 || kv_sslot < 0 || kv_shead < 0 || o_srow < 0 || o_shead < 0)
        return WA_EARG;
    if (!head_shape_ok(hq, hkv, d)) return WA_EUNSUPPORTED;
    if (!window_ok(w)) return WA_EARG;
    if (w->p32 != WA_P_BF16 && w->p32 != WA_P_TWO && w->p32 != WA_P_THREE) return WA_EUNSUPPORTED;
    if ((int64_t)p0 + n > 0x7FFFFFFF || (int64_t)n + w->window > 0x3FFFFFFF) return WA_ERANGE;
    const int64_t first = w->window > 0 ? (int64_t)(p0 - w->window + 1 > 0 ? p0 - w->window + 1 : 0) : 0;
    if ((int64_t)w->ring < (int64_t)p0 + n - first) return WA_ERANGE;
    if (!prompt_extent_ok(kv_sslot, d)) return WA_ERANGE;
    if (((uintptr_t)q | (uintptr_t)k | (uintptr_t)v) & 15) return WA_EARG;
    if ((q_srow | q_shead | kv_sslot | kv_shead) & 7) return WA_EARG;
    if (((uintptr_t)out & 7) || ((o_srow | o_shead) & 3)) return WA_EARG;

    wa::PromptArgs a{};
    a.q = q; a.q_srow = q_srow; a.q_shead = q_shead;
    a.k = k; a.v = v; a.kv_sslot = kv_sslot; a.kv_shead = kv_shead;
    a.p0 = p0; a.n = n; a.hq = hq; a.hkv = hkv; a.d = d;
    a.window = w->window; a.ring = w->ring; a.scale = w->scale; a.p_parts = 1 + w->p32;
    a.ring_magic = wa::mod_magic((uint32_t)w->ring);
    a.hi = hi;
    a.out = out; a.o_srow = o_srow; a.o_shead = o_shead;
    a.nchunk = 1; a.Cp = 0; a.chunk_keys = wa::kPromptChunk; a.pm = a.pl = a.po = nullptr;
    if (w->window > 0) {
        const size_t need = wa_prompt_workspace(w, n, hq, d);
        if (!ws || ws_bytes < need || ((uintptr_t)ws & 15)) return WA_EWORKSPACE;
        a.nchunk = wa::prompt_wg_chunks(w->window, n);
        a.Cp = wa::prompt_pair_chunks(w->window, n);
        const size_t cells = (size_t)n * hq * a.Cp;
        a.pm = static_cast<float*>(ws);
        a.pl = a.pm + cells;
        a.po = a.pl + cells;
        // 16-byte stores of the O partials: the O block starts 16-byte aligned when
        // 2 * cells floats are a multiple of 4, otherwise shift it
        if (((uintptr_t)a.po) & 15) a.po = reinterpret_cast<float*>(((uintptr_t)a.po + 15) & ~(uintptr_t)15);
    }
    if (wa::launch_prompt(a, static_cast<hipStream_t>(stream)) != hipSuccess) return WA_EHIP;
    return WA_OK;
}

size_t wa_prompt_sparse_workspace(const wa_window_t* w, int32_t p0, int32_t n, int32_t hq, int32_t d) {
    if (!window_ok(w) || p0 < 0 || n <= 0 || hq <= 0 || (d != 128 && d != 256)) return 0;
    if ((int64_t)p0 + n > 0x7FFFFFFF) return 0;
    const size_t cells = (size_t)n * (size_t)hq * (size_t)wa::sparse_chunks(w->window, p0, n);
    return cells * sizeof(float) * (2 + (size_t)d) + 16;
}

int wa_prompt_sparse(const wa_window_t* w,
                     const uint16_t* q, int64_t q_srow, int64_t q_shead,
                     const uint16_t* k, const uint16_t* v, int64_t kv_sslot, int64_t kv_shead,
                     int32_t p0, int32_t n, int32_t hq, int32_t hkv, int32_t d,
                     const int32_t* hi, const uint32_t* blocks, int64_t blocks_srow, int32_t blocks_words,
                     void* ws, size_t ws_bytes,
                     uint16_t* out, int64_t o_srow, int64_t o_shead, void* stream) {
    if (!blocks || blocks_words <= 0 || blocks_srow < blocks_words) return WA_EARG;
    if ((uintptr_t)blocks & 3) return WA_EARG;
    if (!w || !q || !k || !v || !out) return WA_EARG;
    if (n <= 0 || p0 < 0) return WA_EARG;
    if (q_srow < 0 || q_shead < 0 || kv_sslot < 0 || kv_shead < 0 || o_srow < 0 || o_shead < 0)
        return WA_EARG;
    if (!head_shape_ok(hq, hkv, d)) return WA_EUNSUPPORTED;
    if (!window_ok(w)) return WA_EARG;
    if (w->p32 != WA_P_BF16 && w->p32 != WA_P_TWO && w->p32 != WA_P_THREE) return WA_EUNSUPPORTED;
    if ((int64_t)p0 + n > 0x7FFFFFFF || (int64_t)n + w->window > 0x3FFFFFFF) return WA_ERANGE;
    const int64_t first = w->window > 0 ? (int64_t)(p0 - w->window + 1 > 0 ? p0 - w->window + 1 : 0) : 0;
    if ((int64_t)w->ring < (int64_t)p0 + n - first) return WA_ERANGE;
    if (!prompt_extent_ok(kv_sslot, d)) return WA_ERANGE;
    if (((uintptr_t)q | (uintptr_t)k | (uintptr_t)v) & 15) return WA_EARG;
    if ((q_srow | q_shead | kv_sslot | kv_shead) & 7) return WA_EARG;
    if (((uintptr_t)out & 7) || ((o_srow | o_shead) & 3)) return WA_EARG;
    const size_t need = wa_prompt_sparse_workspace(w, p0, n, hq, d);
    if (!ws || ws_bytes < need || ((uintptr_t)ws & 15)) return WA_EWORKSPACE;

    wa::PromptArgs a{};
    a.q = q; a.q_srow = q_srow; a.q_shead = q_shead;
    a.k = k; a.v = v; a.kv_sslot = kv_sslot; a.kv_shead = kv_shead;
    a.p0 = p0; a.n = n; a.hq = hq; a.hkv = hkv; a.d = d;
    a.window = w->window; a.ring = w->ring; a.scale = w->scale; a.p_parts = 1 + w->p32;
    a.ring_magic = wa::mod_magic((uint32_t)w->ring);
    a.hi = hi;
    a.out = out; a.o_srow = o_srow; a.o_shead = o_shead;
    a.bm = blocks; a.bm_srow = blocks_srow; a.bm_words = blocks_words;
    a.nchunk = wa::sparse_chunks(w->window, p0, n);
    a.Cp = a.nchunk;
    a.chunk_keys = wa::kPromptChunk;
    const size_t cells = (size_t)n * hq * a.Cp;
    a.pm = static_cast<float*>(ws);
    a.pl = a.pm + cells;
    a.po = a.pl + cells;
    if (((uintptr_t)a.po) & 15) a.po = reinterpret_cast<float*>(((uintptr_t)a.po + 15) & ~(uintptr_t)15);
    if (wa::launch_prompt(a, static_cast<hipStream_t>(stream)) != hipSuccess) return WA_EHIP;
    return WA_OK;
}

int wa_prepare(const wa_prep_t* p,
               const uint16_t* x, int64_t x_srow, int64_t x_shead,
               const int32_t* pos_of_row, const float* qs,
               int32_t rows, int32_t heads, int32_t d,
               const int32_t* stream_of_row, int32_t streams, int32_t ring,
               uint16_t* out, int64_t o_sstream, int64_t o_sslot, int64_t o_shead, void* stream) {
    if (!p || !x || !pos_of_row || !out) return WA_EARG;
    if (rows <= 0 || heads <= 0 || x_srow < 0 || x_shead < 0 || o_sslot < 0 || o_shead < 0 ||
        o_sstream < 0 || ring < 0)
        return WA_EARG;
    if (d != 128 && d != 256) return WA_EUNSUPPORTED;
    if (p->mode != WA_PREP_COPY && p->mode != WA_PREP_ROPE_L2 && p->mode != WA_PREP_RMS_ROPE) return WA_EARG;
    if (p->mode != WA_PREP_COPY) {
        if (p->rope_dims < 0 || p->rope_dims > d || (p->rope_dims & 1)) return WA_EARG;
        if (!(p->theta > 0.f) || !(p->eps >= 0.f)) return WA_EARG;
    }
    if (qs && p->mode != WA_PREP_ROPE_L2) return WA_EARG;
    if (ring > 0 && (!stream_of_row || streams <= 0)) return WA_EARG;
    // 4- or 8-byte lane accesses (d / 64 bf16 a lane)
    const uintptr_t al = (uintptr_t)(d / 32);
    if (((uintptr_t)x | (uintptr_t)out) & (al - 1)) return WA_EARG;
    if ((x_srow | x_shead | o_sstream | o_sslot | o_shead) & (int64_t)(al / 2 - 1)) return WA_EARG;
    if (qs && ((uintptr_t)qs & 3)) return WA_EARG;
    wa::PrepArgs a{};
    // a copy rotates nothing: its rope_dims is not checked above and must not index the
    // kernels' cos/sin table
    a.mode = p->mode; a.rope_dims = p->mode == WA_PREP_COPY ? 0 : p->rope_dims;
    a.theta = p->theta; a.eps = p->eps;
    // the inverse frequencies depend on j only: computed once here, in float64 and rounded
    // once to fp32, instead of on every row of the kernel
    if (p->mode != WA_PREP_COPY)
        for (int j = 0; j < p->rope_dims / 2; ++j)
            a.inv[j] = (float)std::pow((double)p->theta, -2.0 * (double)j / (double)p->rope_dims);
    a.x = x; a.x_srow = x_srow; a.x_shead = x_shead;
    a.pos_of_row = pos_of_row; a.qs = qs;
    a.rows = rows; a.heads = heads; a.d = d;
    a.stream_of_row = stream_of_row; a.streams = streams; a.ring = ring;
    a.out = out; a.o_sstream = o_sstream; a.o_sslot = o_sslot; a.o_shead = o_shead;
    if (wa::launch_prepare(a, static_cast<hipStream_t>(stream)) != hipSuccess) return WA_EHIP;
    return WA_OK;
}

const char* wa_status_string(int status) {
    switch (status) {
        case WA_OK: return "ok";
        case WA_EARG: return "invalid argument";
        case WA_EUNSUPPORTED: return "unsupported shape";
        case WA_ERANGE: return "window or ring inconsistent with the positions";
        case WA_EWORKSPACE: return "workspace missing or too small";
        case WA_EHIP: return "kernel launch failed";
        case WA_ESCRATCH: return "call needs more than wa_decode_noalloc's static scratch";
        default: return "unknown status";
    }
}

const char* wa_version(void) { return "wa 0.1 gfx950"; }

}  // extern "C"
