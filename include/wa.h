/*
 * wa.h -- windowed grouped-query softmax attention on MI355X (gfx950), C ABI.
 *
 * The operation (TensorFold pull request #1123, "window_attention at head dim 256",
 * section "What this changes"): for each query row i at key position p_i and each query
 * head h, with key head g = h / G (G = hq / hkv query heads per key head, any G up to 16),
 *
 *     visible keys   j in [lo_i, last_i],  lo_i = max(0, p_i - window + 1)  (0 if window == 0)
 *     score          s_j  = scale * (q_i,h . k_j,g)
 *     output         o_i,h = sum_j softmax(s)_j v_j,g, rounded once to bf16 (nearest-even)
 *
 * last_i is the row's own position, or hi[i] in the prompt form ("promptRows(..., hi)"
 * bullet). Key j is stored in ring slot j mod ring ("Scale/Window 0" bullet; window 0
 * means a linear cache, i.e. a ring as long as the cache).
 *
 * Two forms:
 *   decode  split-KV over 256-key chunks at absolute key positions, per-chunk partials
 *           (m_c, l_c, o_c) in fp32 with fp32 probabilities, then a merge over the chunks in
 *           chunk order ("Decode" bullet). A row's bits do not depend on the batch, the
 *           stream slot or the declared cache length.
 *   prompt  rows p0 .. p0+n-1 of one stream, tiled online softmax on MFMA (bf16 products,
 *           fp32 accumulation), key tiles at absolute positions ("Prompt" bullet); P enters
 *           P.V as one bf16, or with p32 as bf16(P) + bf16(P - bf16(P)) ("Window.p32" bullet),
 *           or as three bf16 parts that sum to P exactly (WA_P_THREE).
 *           Windowed prompts are also split into 384-key chunks merged in chunk order.
 *           A row's bits do not depend on how the prompt is chunked.
 *
 * Conventions for every entry point:
 *   - bf16 tensors are passed as uint16_t bit patterns; every tensor pointer is a DEVICE
 *     pointer; strides are in elements; the innermost (dim) stride is 1.
 *   - q/out are [rows][hq][d] with row and head strides; the K and V caches share one layout
 *     [stream][slot][kv head][d] with stream, slot and head strides.
 *   - d is 128 or 256; hq % hkv == 0 and hq / hkv <= 16.
 *   - The library allocates, frees and synchronises nothing, and keeps no per-call state; it
 *     is safe to call from several host threads. Work is queued on `stream` (a hipStream_t;
 *     NULL is the default stream). Inputs must stay alive and unchanged, and outputs must not
 *     be read, until that stream has completed the call.
 *   - Host-checkable mistakes return a negative status and launch nothing. Device-side
 *     preconditions (positions, stream indices, hi) cannot be checked without a
 *     synchronisation; the kernels clamp them into range so that every access stays inside
 *     the caller's buffers, and the result for a violating row is then unspecified.
 *   - Non-finite outputs take float64's class: wa_decode and wa_prompt re-run, in float64,
 *     exactly the (row, head)s whose bf16 output holds a NaN or an infinity (the pull
 *     request's non-finite bullet and review: per row and head, never per block). fp32 can
 *     differ from float64 only there (a weight that underflows to 0 beside an infinite value,
 *     0 * inf in a shared MFMA tile, fp32 overflow of q . k). wa_merge alone does not re-run
 *     (it has no q, K, V).
 */
#ifndef WA_H
#define WA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Window parameters shared by both forms ("Window" in the pull request). */
typedef struct wa_window {
    int32_t window;  /* keys a row sees up to its last key; 0 = no window (linear cache) */
    int32_t ring;    /* slots per stream in the K/V cache (the cache length when window == 0) */
    float   scale;   /* score scale: s = scale * (q . k) */
    int32_t p32;     /* prompt only: how P enters P.V, one of WA_P_* below */
} wa_window_t;

/* Values of wa_window_t.p32 (the prompt's representation of the fp32 probabilities P in the
 * bf16 P.V product; fp32 accumulation in every case):
 *   WA_P_BF16   one bf16, bf16(P) (relative error up to 2^-8)               "Window.p32" off
 *   WA_P_TWO    two parts, bf16(P) + bf16(P - bf16(P)) (P to 2^-16)           "Window.p32" on
 *   WA_P_THREE  three parts hi + mid + lo, each the bf16 rounding of what the earlier parts
 *               leave; their sum is P exactly (P >= 2^-110), so the P.V products are those of
 *               fp32 P (the three-part 16-bit split of TensorFold pull request #1622, review
 *               answer, "What changed"); P.V costs three MFMA passes.
 * Other values: WA_EUNSUPPORTED. */
enum { WA_P_BF16 = 0, WA_P_TWO = 1, WA_P_THREE = 2 };

enum {
    WA_OK = 0,
    WA_EARG = -1,          /* null pointer, non-positive size, bad stride */
    WA_EUNSUPPORTED = -2,  /* head dim other than 128/256, hq % hkv != 0, group > 16 */
    WA_ERANGE = -3,        /* window/ring inconsistent with the positions the call can reach */
    WA_EWORKSPACE = -4,    /* decode workspace missing or smaller than wa_decode_workspace() */
    WA_EHIP = -5,          /* a kernel launch failed (hipGetLastError after the launch) */
    WA_ESCRATCH = -6       /* wa_decode_noalloc: the call needs more than its static scratch */
};

/* Most chunks a decode row can span: window > 0: (window - 1 + 255) / 256 + 1;
 * window == 0: max_pos / 256 + 1. Returns 0 for invalid arguments. */
int32_t wa_decode_chunks(const wa_window_t* w, int32_t max_pos);

/* Bytes of device workspace wa_decode needs for `rows` rows of `hq` heads of dim `d`:
 * fp32 partials m, l [rows][hq][C] and o [rows][hq][C][d], C = wa_decode_chunks(). With
 * cells = rows * hq * C rounded up to even, m starts at the workspace, l at float offset
 * cells and o at float offset 2 * cells (so o is 16-byte aligned, as wa_merge needs).
 * 0 on error. */
size_t wa_decode_workspace(int32_t rows, int32_t hq, int32_t d, const wa_window_t* w,
                           int32_t max_pos);

/*
 * Decode: row r (0 <= r < rows) of stream stream_of_row[r] at position pos_of_row[r] (both
 * device int32 arrays) attends over keys [lo_r, pos_r] of its stream's ring. Launches the
 * chunk-partial kernel (one workgroup per (row, key head, chunk)) and the ordered merge.
 *   q        [rows][hq][d]          strides q_srow, q_shead
 *   k, v     [streams][ring][hkv][d] strides kv_sstream, kv_sslot, kv_shead
 *   max_pos  an upper bound of every pos_of_row[r] (sizes the chunk grid when window == 0)
 *   ws       device workspace, 16-byte aligned, of ws_bytes >= wa_decode_workspace(rows, hq,
 *            d, w, max_pos); after the call it holds the chunk partials in the layout above
 *   out      [rows][hq][d]          strides o_srow, o_shead
 * Device preconditions: 0 <= pos_of_row[r] <= max_pos, 0 <= stream_of_row[r] < streams, and
 * the ring holds keys [lo_r, pos_r] of row r's stream in slots j mod ring. Errors: WA_EARG,
 * WA_EUNSUPPORTED, WA_ERANGE (window > ring, window == 0 and max_pos >= ring, or a key head's
 * ring spanning 2^31 bytes or more: (ring - 1) * kv_sslot * 2 + 2 * d >= 2^31 - 1),
 * WA_EWORKSPACE, WA_EHIP.
 */
int wa_decode(const wa_window_t* w,
              const uint16_t* q, int64_t q_srow, int64_t q_shead,
              const uint16_t* k, const uint16_t* v,
              int64_t kv_sstream, int64_t kv_sslot, int64_t kv_shead, int32_t streams,
              const int32_t* stream_of_row, const int32_t* pos_of_row, int32_t max_pos,
              int32_t rows, int32_t hq, int32_t hkv, int32_t d,
              void* ws, size_t ws_bytes,
              uint16_t* out, int64_t o_srow, int64_t o_shead, void* stream);

/*
 * Decode for callers that cannot allocate device memory (code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc): wa_decode with the same arguments except
 * the workspace, whose role a static device array of WA_NOALLOC_SCRATCH_BYTES (8 MiB) takes.
 * Each GPU the library runs on holds its own copy of that array from the first call on that
 * device until the process ends; the call allocates and frees nothing. Results are wa_decode's
 * bits. A call whose wa_decode_workspace() size exceeds WA_NOALLOC_SCRATCH_BYTES returns
 * WA_ESCRATCH and launches nothing (8 MiB holds the partials of, e.g., 101 rows of 16 heads x
 * 256 over 5 chunks). Every call on one GPU uses that GPU's one array and leaves its partials
 * there: calls that may overlap on one GPU (other streams, other host threads) race and must
 * be serialised by the caller. Other errors as wa_decode (WA_EHIP also if the array's device
 * address cannot be queried).
 */
#define WA_NOALLOC_SCRATCH_BYTES ((size_t)8 << 20)
int wa_decode_noalloc(const wa_window_t* w,
                      const uint16_t* q, int64_t q_srow, int64_t q_shead,
                      const uint16_t* k, const uint16_t* v,
                      int64_t kv_sstream, int64_t kv_sslot, int64_t kv_shead, int32_t streams,
                      const int32_t* stream_of_row, const int32_t* pos_of_row, int32_t max_pos,
                      int32_t rows, int32_t hq, int32_t hkv, int32_t d,
                      uint16_t* out, int64_t o_srow, int64_t o_shead, void* stream);

/*
 * Merge of decode partials (the second half of wa_decode, exposed so that partials made
 * elsewhere, e.g. gathered from several devices, can be combined with the same bits).
 * For row r and head h it reads chunks c = 0 .. n_r - 1 of the partial arrays, where n_r is
 * the number of 256-key chunks holding keys [lo_r, pos_r] (pos from pos_of_row), in chunk
 * order: M = max m_c, a_c = exp(m_c - M), out = bf16(sum a_c o_c / sum a_c l_c), both sums
 * fma chains over the chunks in order ("Decode" bullet of the pull request).
 *   m, l  [rows][hq][C] fp32      o  [rows][hq][C][d] fp32 (16-byte aligned)   C = chunk capacity
 * Device precondition: n_r <= C (rows violating it read only their first C chunks).
 * Errors: WA_EARG (also for an o that is not 16-byte aligned), WA_EUNSUPPORTED, WA_EHIP.
 */
int wa_merge(const wa_window_t* w, const float* m, const float* l, const float* o,
             const int32_t* pos_of_row, int32_t rows, int32_t hq, int32_t C, int32_t d,
             uint16_t* out, int64_t o_srow, int64_t o_shead, void* stream);

/* Bytes of device workspace wa_prompt needs: 0 for window == 0; otherwise fp32 partials
 * m, l [n][hq][Cp] and o [n][hq][Cp][d] with Cp = (window - 1 + n) / 384 + 2, plus 16 bytes
 * of alignment slack. 0 on invalid arguments (and for window == 0). */
size_t wa_prompt_workspace(const wa_window_t* w, int32_t n, int32_t hq, int32_t d);

/*
 * Prompt: rows i = 0 .. n-1 at positions p0 + i of one stream. Row i sees keys
 * [lo_i, last_i] with last_i = hi[i] if hi is not NULL (device int32 [n],
 * p0 + i <= hi[i] < p0 + n), else p0 + i.
 *   q        [n][hq][d]       strides q_srow, q_shead
 *   k, v     [ring][hkv][d]   strides kv_sslot, kv_shead (one stream's ring)
 *   ws       device workspace, 16-byte aligned, of ws_bytes >= wa_prompt_workspace(w, n, hq, d)
 *            (may be NULL when window == 0)
 *   out      [n][hq][d]       strides o_srow, o_shead
 * With a window (> 0) the keys of every row are split into 384-key chunks at absolute
 * positions: one tiled online softmax per chunk gives fp32 partials (m in log2 units, l, O),
 * and a merge combines a row's chunks in chunk order (the decode's split applied to the
 * prompt, so that short windowed prompts fill the GPU); window 0 runs one online softmax over
 * the row's whole key range. Either way a row's bits depend only on its own keys and the
 * absolute chunk and tile grid, not on how the prompt is cut into calls.
 * The ring must hold keys [min lo_i, p0 + n - 1] without two of them sharing a slot:
 * ring >= p0 + n - max(0, p0 - window + 1) (window > 0) or ring >= p0 + n (window == 0),
 * else WA_ERANGE. A 64-key tile of a key head is addressed with 32-bit byte offsets:
 * 63 * kv_sslot * 2 + 2 * d >= 2^31 - 1 is also WA_ERANGE.
 * hi values out of range are clamped into [p0 + i, p0 + n - 1].
 * w->p32 selects P's representation (WA_P_*; another value is WA_EUNSUPPORTED).
 * Errors: WA_EARG, WA_EUNSUPPORTED, WA_ERANGE, WA_EWORKSPACE, WA_EHIP.
 */
int wa_prompt(const wa_window_t* w,
              const uint16_t* q, int64_t q_srow, int64_t q_shead,
              const uint16_t* k, const uint16_t* v, int64_t kv_sslot, int64_t kv_shead,
              int32_t p0, int32_t n, int32_t hq, int32_t hkv, int32_t d,
              const int32_t* hi, void* ws, size_t ws_bytes,
              uint16_t* out, int64_t o_srow, int64_t o_shead, void* stream);

/* Bytes of device workspace wa_prompt_sparse needs: fp32 partials m, l [n][hq][Cs] and
 * o [n][hq][Cs][d], Cs = (window - 1 + n) / 384 + 2 with a window, (p0 + n - 1) / 384 + 1
 * without, plus 16 bytes of alignment slack. 0 on invalid arguments. */
size_t wa_prompt_sparse_workspace(const wa_window_t* w, int32_t p0, int32_t n, int32_t hq, int32_t d);

/*
 * Block-sparse prompt (TensorFold pull request #1622, "What this changes": per-row block
 * masks over the union of a row group's selected blocks, causal ends, fp32 online softmax,
 * the parts/merge layout). Row i sees the keys j of its wa_prompt range [lo_i, last_i]
 * whose 64-key block b = j / 64 is selected: bit b % 32 of blocks[i * blocks_srow + b / 32]
 * (device uint32, 4-byte aligned; words at or past blocks_words count as zero). Everything
 * else is wa_prompt's: arguments, ring rule, hi, w->p32 (WA_P_*), and the 384-key chunks at
 * absolute positions merged in chunk order, where a chunk holding none of a row's keys takes
 * no part. A workgroup of rows walks the union of their selected tiles; each row masks the
 * blocks it did not select, so its bits depend only on its own keys (equal to wa_prompt's
 * with every block selected and a window > 0). A row that sees no key gets NaN (0 / 0).
 * Errors: WA_EARG (also blocks NULL, blocks_words <= 0, blocks_srow < blocks_words),
 * WA_EUNSUPPORTED, WA_ERANGE, WA_EWORKSPACE (ws smaller than wa_prompt_sparse_workspace),
 * WA_EHIP.
 */
int wa_prompt_sparse(const wa_window_t* w,
                     const uint16_t* q, int64_t q_srow, int64_t q_shead,
                     const uint16_t* k, const uint16_t* v, int64_t kv_sslot, int64_t kv_shead,
                     int32_t p0, int32_t n, int32_t hq, int32_t hkv, int32_t d,
                     const int32_t* hi, const uint32_t* blocks, int64_t blocks_srow,
                     int32_t blocks_words, void* ws, size_t ws_bytes,
                     uint16_t* out, int64_t o_srow, int64_t o_shead, void* stream);

/* q/k row preparation, the step before the attention (TensorFold pull request #1257,
 * "What this changes"; the "Exact Numerical Contract" page, "Preparation"). */
enum {
    WA_PREP_COPY = 0,      /* the row as it is (values into the cache) */
    WA_PREP_ROPE_L2 = 1,   /* r = bf16(rope(x)), n = bf16(r / sqrt(sum r^2 + eps)),
                              then q = bf16(qs * n) when qs is given (fp32 cos/sin) */
    WA_PREP_RMS_ROPE = 2   /* n = bf16(x / sqrt(mean x^2 + eps)), r = bf16(rope(n)) with
                              bf16 cos/sin coefficients */
};
typedef struct wa_prep {
    int32_t mode;       /* WA_PREP_* */
    int32_t rope_dims;  /* R: even, 0 <= R <= d; rotate-half over dims 0..R-1, pairs (j, j+R/2) */
    float   theta;      /* RoPE base: inv_j = fl32(theta^(-2j/R)), angle fl32(fl32(pos) * inv_j) */
    float   eps;        /* the pages' values: 1e-6 on the sum (L2), 1e-5 on the mean (RMS) */
} wa_prep_t;

/*
 * Prepare rows r = 0 .. rows-1 (position pos_of_row[r], device int32) of `heads` heads:
 *   x    [rows][heads][d] bf16, strides x_srow, x_shead (the projection's rows)
 *   qs   fp32 [d] (device) or NULL: q scale of WA_PREP_ROPE_L2 (rejected in other modes)
 *   out  ring == 0: row r at out + r * o_sslot (+ head * o_shead);
 *        ring  > 0: row r into the cache slot pos mod ring of stream stream_of_row[r]:
 *                   out + stream * o_sstream + (pos mod ring) * o_sslot + head * o_shead
 * cos and sin are the fp32 values of the angle's cosine and sine, correctly rounded
 * (within the page's 2-ulp cosf/sinf); all other arithmetic is fp32 and every rounding
 * point named in the mode rounds to bf16, nearest-even.
 * Device preconditions: pos >= 0 (negative values are taken as 0), 0 <= stream_of_row[r]
 * < streams (clamped). x and out 8-byte aligned (4-byte at d = 128), strides multiples of 4
 * (2 at d = 128); with x and out 16-byte aligned, strides multiples of 8 and rope_dims a
 * multiple of 16 (or a copy) the call takes a faster form (16-byte accesses), same results
 * within the stated roundings. Errors: WA_EARG, WA_EUNSUPPORTED (d other than 128 or 256),
 * WA_EHIP.
 */
int wa_prepare(const wa_prep_t* p,
               const uint16_t* x, int64_t x_srow, int64_t x_shead,
               const int32_t* pos_of_row, const float* qs,
               int32_t rows, int32_t heads, int32_t d,
               const int32_t* stream_of_row, int32_t streams, int32_t ring,
               uint16_t* out, int64_t o_sstream, int64_t o_sslot, int64_t o_shead, void* stream);

/* Human-readable name of a status code (static storage). */
const char* wa_status_string(int status);

/* Library version string (static storage). */
const char* wa_version(void);

#ifdef __cplusplus
}
#endif

#endif /* WA_H */
