/*
 * kvc.h -- C ABI of libkvc, an MI355X (gfx950) KV-cache codec in the style of
 * CacheGen ("CacheGen: KV Cache Compression and Streaming for Fast Large
 * Language Model Serving", SIGCOMM 2024; wiki summary page, section 核心方法).
 *
 * The page's pipeline: split the KV cache along tokens into chunks of about
 * 1.5K tokens; inside a chunk, group tokens by 10 with the first token as an
 * 8-bit anchor and the others as deltas to it; quantize deltas more coarsely
 * for deeper thirds of the layers; arithmetic-code the symbols against
 * distributions profiled offline per channel-layer combination (anchors and
 * deltas separately); store each chunk at several compression levels; on
 * restore, fetch chunks, decode them on the GPU and concatenate them into the
 * KV cache.  The exact numeric definitions used here (quantizers, range
 * coder, container layout, profile id) are the ones written out in the
 * project's design notes; all entry points below follow them.
 *
 * Conventions (all entry points):
 *  - Tensor arguments are DEVICE pointers owned by the caller; host arrays are
 *    marked "host".  The library never allocates or frees device memory and
 *    keeps no device state between calls: scratch space is the caller's
 *    workspace `ws` of at least the size returned by the matching *_ws_bytes
 *    query (any alignment of 256 bytes or more).
 *  - Every call is asynchronous on `stream` (a hipStream_t, e.g. torch's
 *    current stream).  Argument and shape errors are returned synchronously
 *    before anything is launched or written.
 *  - Errors found on the device (corrupt bitstream, profile mismatch,
 *    non-finite input, output capacity) are written to the caller's device
 *    word `*dev_status`: each call first sets it to 0 (stream-ordered), then
 *    the first error code seen (a negative kvc_status) replaces the 0.  Read
 *    it after synchronizing the stream.  On such an error the contents of the
 *    output are unspecified, but nothing outside the output and `ws` is
 *    written.
 *  - KV layout: binary16 bit patterns in [layer][K=0,V=1][token][channel],
 *    channel fastest; C channels per K and per V (kv_heads * head_dim).
 *  - Calls on distinct workspaces may run concurrently; calls sharing a
 *    workspace must be ordered on one stream.
 */
#ifndef KVC_H_
#define KVC_H_

#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  KVC_OK = 0,
  KVC_ERR_INVALID_ARG = -1,     /* bad descriptor, null pointer, bad level */
  KVC_ERR_SHAPE = -2,           /* token ranges / sizes inconsistent */
  KVC_ERR_PROFILE_MISMATCH = -3,/* container made with other tables */
  KVC_ERR_CORRUPT_STREAM = -4,  /* bad header, bad lengths, undecodable bytes */
  KVC_ERR_NONFINITE = -5,       /* inf / NaN in the KV to encode or profile */
  KVC_ERR_CAPACITY = -6,        /* workspace or output buffer too small */
  KVC_ERR_HIP = -7,             /* a HIP runtime call failed */
  KVC_ERR_UNIMPLEMENTED = -8     /* no entry point returns it */
} kvc_status;

/* Codec descriptor: the page's constants (chunks of ~1.5K tokens, groups of
 * 10 tokens, 8-bit anchors, coarser deltas for deeper layer thirds).
 * Supported: group_tokens in [1, chunk_tokens], anchor_bits == 8,
 * cdf_prec_bits == 15, n_levels in [1, 4], delta_bits in [2, 6]. */
typedef struct {
  uint32_t n_layers;         /* L >= 1 */
  uint32_t n_channels;       /* C >= 1, per K and per V */
  uint32_t group_tokens;     /* 10 */
  uint32_t chunk_tokens;     /* 1500 */
  uint32_t anchor_bits;      /* 8 */
  uint32_t n_levels;         /* compression levels held by the tables */
  uint8_t delta_bits[4][3];  /* [level][layer third], third(l) = 3l / L */
  uint32_t cdf_prec_bits;    /* 15 */
} kvc_codec_desc;

/* One encoded chunk handed to the decoder (a fetched bitstream). */
typedef struct {
  const uint8_t *container; /* device pointer to the chunk's container */
  uint64_t container_bytes; /* its size in bytes */
  uint32_t first_token;     /* destination token offset in kv_out */
  uint32_t n_tokens;        /* tokens in the chunk; must equal the header */
  uint32_t level;           /* compression level; must equal the header */
  uint32_t reserved;        /* 0 */
} kvc_chunk_ref;

/* One encoded chunk of one of several requests, for kvc_decode_multi: the
 * fields of kvc_chunk_ref plus the request's own KV cache. */
typedef struct {
  const uint8_t *container; /* device pointer to the chunk's container */
  uint64_t container_bytes; /* its size in bytes */
  uint32_t first_token;     /* destination token offset in kv_out */
  uint32_t n_tokens;        /* tokens in the chunk; must equal the header */
  uint32_t level;           /* compression level; must equal the header */
  uint32_t reserved;        /* 0 */
  uint16_t *kv_out;         /* device: the request's KV cache [L][2][T_total][C] */
  uint32_t T_total;         /* its token capacity */
  uint32_t reserved2;       /* 0 */
} kvc_request_chunk;

/* One encoded chunk still in host memory, for kvc_restore. */
typedef struct {
  const uint8_t *host_container; /* host pointer; pinned (hipHostMalloc) memory
                                    lets the copy overlap the decode */
  uint64_t container_bytes;      /* its size in bytes */
  uint32_t first_token;          /* destination token offset in kv_out */
  uint32_t n_tokens;             /* tokens in the chunk; must equal the header */
  uint32_t level;                /* compression level; must equal the header */
  uint32_t reserved;             /* 0 */
} kvc_host_chunk;

/* One chunk's base container and its refinement container, for
 * kvc_decode_refined. */
typedef struct {
  const uint8_t *container;  /* device pointer to the chunk's base container */
  uint64_t container_bytes;  /* its size in bytes */
  const uint8_t *refinement; /* device pointer to the chunk's refinement container */
  uint64_t refinement_bytes; /* its size in bytes */
  uint32_t first_token;      /* destination token offset in kv_out */
  uint32_t n_tokens;         /* tokens in the chunk; must equal both headers */
  uint32_t level;            /* base level; must equal both headers */
  uint32_t reserved;         /* 0 */
} kvc_refined_chunk_ref;

/* Library version (major * 10000 + minor * 100 + patch). */
int kvc_version(void);

/* Human-readable name of a status code (static string). */
const char *kvc_status_str(kvc_status s);

/* KVC_OK if the descriptor is supported, else KVC_ERR_INVALID_ARG. */
kvc_status kvc_validate_desc(const kvc_codec_desc *d);

/* ---------------------------------------------------------------- tables */
/* Size in bytes of the profiled tables blob: a 128-byte header, then the
 * anchor cumulative frequencies [2LC][264] u16, then the delta cumulative
 * frequencies [n_levels][2LC][64] u16.  0 if the descriptor is invalid. */
uint64_t kvc_tables_bytes(const kvc_codec_desc *d);

/* Workspace bytes needed by kvc_profile. */
uint64_t kvc_profile_ws_bytes(const kvc_codec_desc *d);

/*
 * Offline profiling (CacheGen page, 核心方法 step 3 and 关键观察 observation
 * 3: distributions profiled per channel-layer combination and reused across
 * contexts of the same model).  kv_fp16: profiling KV [L][2][T][C]; it is
 * split into chunks of chunk_tokens and every chunk is quantized (anchors
 * once, deltas once per level); symbol counts are normalised to 2^15 per
 * model.  Writes the tables blob (kvc_tables_bytes bytes) including its
 * 64-bit profile id.  Device errors: KVC_ERR_NONFINITE.
 */
kvc_status kvc_profile(const kvc_codec_desc *d, const uint16_t *kv_fp16, uint32_t T,
                       void *tables_out, void *ws, uint64_t ws_bytes, int32_t *dev_status,
                       hipStream_t stream);

/* ---------------------------------------------------------------- encode */
/* Upper bound of one chunk's container for n_tokens tokens. */
uint64_t kvc_container_bound(const kvc_codec_desc *d, uint32_t n_tokens);

/* Upper bound of all containers of a T-token context (sum over chunks). */
uint64_t kvc_encode_bound(const kvc_codec_desc *d, uint32_t T);

/* Workspace bytes needed by kvc_encode for a T-token context. */
uint64_t kvc_encode_ws_bytes(const kvc_codec_desc *d, uint32_t T);

/*
 * Encode a T-token KV cache (CacheGen page, 核心方法 steps 1-3: chunking,
 * change-based anchor/delta encoding, layer-wise quantization, arithmetic
 * coding).  Chunk k = tokens [k*chunk_tokens, ...) is coded at level
 * chunk_levels[k] (host array of ceil(T / chunk_tokens) entries) into one
 * container; containers are written back to back into `out` (device,
 * out_cap bytes) and chunk_offsets_out (device, n_chunks + 1 u64) receives
 * each container's start offset and, last, the total size.
 * Each container's payload holds, per unit of up to 64 consecutive streams
 * of one (layer, K/V) row, the streams' 8-byte blocks in the order in which
 * the decoder's 64 lanes ask for them while decoding (so that one wave's
 * requests are consecutive bytes); a stream's block padding is zero.
 * Every valid input is encoded: a range-coder carry may run back through any
 * number of 0xFF bytes already produced (the few (chunk, unit)s where that
 * happens are coded a second time, by a slower kernel).
 * Device errors: KVC_ERR_NONFINITE, KVC_ERR_CAPACITY (out_cap too small; the
 * offsets are still written, `out` is not), KVC_ERR_CORRUPT_STREAM (damaged
 * tables).
 */
kvc_status kvc_encode(const kvc_codec_desc *d, const void *tables, const uint16_t *kv_fp16,
                      uint32_t T, const uint8_t *chunk_levels, uint8_t *out, uint64_t out_cap,
                      uint64_t *chunk_offsets_out, void *ws, uint64_t ws_bytes,
                      int32_t *dev_status, hipStream_t stream);

/* ---------------------------------------------------------------- decode */
/* Workspace bytes needed by kvc_decode / kvc_decode_index for n_chunks. */
uint64_t kvc_decode_ws_bytes(const kvc_codec_desc *d, uint32_t n_chunks);

/*
 * Decode fetched chunks back into the KV cache (CacheGen page, 核心方法: the
 * online side decodes each chunk's bitstream to tensors and concatenates the
 * chunks into the KV cache).  chunks: host array of n_chunks references whose
 * token ranges [first_token, first_token + n_tokens) must be disjoint and
 * inside [0, T_total).  kv_out: device [L][2][T_total][C] binary16; tokens
 * outside the chunks' ranges are not written.  One call runs the bitstream
 * index (per-stream offsets, header checks) and then the fused range-decode /
 * dequantize / store kernel.
 * Device errors: KVC_ERR_PROFILE_MISMATCH, KVC_ERR_CORRUPT_STREAM.
 */
kvc_status kvc_decode(const kvc_codec_desc *d, const void *tables, const kvc_chunk_ref *chunks,
                      uint32_t n_chunks, uint16_t *kv_out, uint32_t T_total, void *ws,
                      uint64_t ws_bytes, int32_t *dev_status, hipStream_t stream);

/*
 * kvc_decode for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc):
 * the same arguments without `ws` / `ws_bytes`, the same kernels and the
 * same results.  Its scratch is a fixed array of
 * KVC_DECODE_STATIC_SCRATCH_BYTES in the library's device memory, one per
 * GPU (the current device's is used; `stream` must belong to that device),
 * held from the first call on a device until the process ends.  The call
 * allocates nothing.  Requests whose kvc_decode workspace
 * (kvc_decode_ws_bytes(d, n_chunks)) is larger than the array return
 * KVC_ERR_CAPACITY before anything is launched.  Every call on one GPU uses
 * the same array: calls that overlap on that GPU (on different streams, or
 * from different host threads without ordering) race and give undefined
 * results; calls ordered on one stream are safe.  Nothing in the array has
 * to start at zero: each call rewrites what it reads.
 * Device errors: those of kvc_decode.
 */
#define KVC_DECODE_STATIC_SCRATCH_BYTES (32ull << 20)
kvc_status kvc_decode_static(const kvc_codec_desc *d, const void *tables,
                             const kvc_chunk_ref *chunks, uint32_t n_chunks, uint16_t *kv_out,
                             uint32_t T_total, int32_t *dev_status, hipStream_t stream);

/*
 * The bitstream index alone: validates the containers' headers against the
 * tables and writes offsets_out (device, [n_chunks][2LC] u32): each stream's
 * byte offset from the start of its container's payload (exclusive prefix
 * sum of the stream lengths rounded up to 8-byte blocks; a unit's blocks
 * start at the offset of its first stream).  Used by kvc_decode; exported
 * for inspection and tests.
 */
kvc_status kvc_decode_index(const kvc_codec_desc *d, const void *tables,
                            const kvc_chunk_ref *chunks, uint32_t n_chunks, uint32_t *offsets_out,
                            void *ws, uint64_t ws_bytes, int32_t *dev_status, hipStream_t stream);

/*
 * Decode chunks of several requests in one call (CacheGen page, 核心方法,
 * online streaming paragraph: with concurrent requests the chunks are
 * batched on the GPU).  Each chunk names its own KV cache; caches of one
 * model share `tables`.  Chunks writing to the same kv_out must agree on
 * T_total and have disjoint token ranges; different caches must not
 * overlap in memory.  No padding: chunks of any lengths and positions mix
 * freely.  Every chunk is decoded exactly as kvc_decode would (same kernels,
 * same bits).  ws: kvc_decode_ws_bytes(d, n_chunks) bytes.
 * Device errors: those of kvc_decode.
 */
kvc_status kvc_decode_multi(const kvc_codec_desc *d, const void *tables,
                            const kvc_request_chunk *chunks, uint32_t n_chunks, void *ws,
                            uint64_t ws_bytes, int32_t *dev_status, hipStream_t stream);

/* ------------------------------------------------- incremental refinement */
/*
 * Incremental, SVC-like refinement (CacheGen page, 局限与 Future Work:
 * low-quality KV first, refinement bits after).  The page gives no scheme;
 * the one here is a second layer per chunk that leaves the base layer (the
 * chunk's container at its level) untouched: per stream it quantizes the
 * residual e = x - xh against the base layer's binary32 reconstruction xh
 * (before its binary16 rounding) with E = refine_bits bits, one scale for
 * the stream's anchor tokens and one for its other tokens (D = max |e| /
 * (2^(E-1) - 1), q = rint(e / D) clamped), and range-codes the symbols
 * against two models per (level, layer, K/V, channel).  A refined value is
 * binary16(fma(q, D, xh)); it lies within D/2 (plus rounding) of the input,
 * about 2^(1-E) of the base layer's error.  Supported: refine_bits in [2, 6].
 */

/* Size in bytes of the refinement tables blob: a 128-byte header, then the
 * anchor-token cumulative frequencies [n_levels][2LC][64] u16, then those
 * of the other tokens.  0 if the descriptor is invalid. */
uint64_t kvc_refine_tables_bytes(const kvc_codec_desc *d);

/* Workspace bytes needed by kvc_profile_refine. */
uint64_t kvc_refine_profile_ws_bytes(const kvc_codec_desc *d);

/*
 * Offline profiling of the refinement models on the profiling KV
 * [L][2][T][C] (chunked like kvc_profile, every level): writes the
 * refinement tables blob (kvc_refine_tables_bytes) with its 64-bit id,
 * which also covers `tables`' profile id (the base tables the refinement
 * goes with).  Device errors: KVC_ERR_NONFINITE.
 */
kvc_status kvc_profile_refine(const kvc_codec_desc *d, const void *tables,
                              const uint16_t *kv_fp16, uint32_t T, uint32_t refine_bits,
                              void *rtables_out, void *ws, uint64_t ws_bytes, int32_t *dev_status,
                              hipStream_t stream);

/* Workspace bytes needed by kvc_encode_refine for a T-token context. */
uint64_t kvc_encode_refine_ws_bytes(const kvc_codec_desc *d, uint32_t T);

/*
 * The refinement layer of a T-token KV cache: chunk k over its base layer at
 * chunk_levels[k] (host array), one refinement container ("KVCR") per chunk,
 * written back to back into `out` (device, out_cap bytes; kvc_encode_bound
 * is enough), with chunk_offsets_out (device, n_chunks + 1 u64) as for
 * kvc_encode.  Its payload uses the same block order as the base containers.
 * Device errors: KVC_ERR_NONFINITE, KVC_ERR_CAPACITY,
 * KVC_ERR_PROFILE_MISMATCH (rtables made for another descriptor or E).
 */
kvc_status kvc_encode_refine(const kvc_codec_desc *d, const void *rtables, uint32_t refine_bits,
                             const uint16_t *kv_fp16, uint32_t T, const uint8_t *chunk_levels,
                             uint8_t *out, uint64_t out_cap, uint64_t *chunk_offsets_out,
                             void *ws, uint64_t ws_bytes, int32_t *dev_status,
                             hipStream_t stream);

/* Workspace bytes needed by kvc_decode_refined for n_chunks. */
uint64_t kvc_decode_refined_ws_bytes(const kvc_codec_desc *d, uint32_t n_chunks);

/*
 * Decode chunks from their base and refinement containers in one launch:
 * every lane decodes a stream's base layer and its refinement layer token by
 * token and writes the refined binary16 values into kv_out
 * [L][2][T_total][C].  Token ranges must be disjoint and inside T_total.
 * Device errors: those of kvc_decode, plus KVC_ERR_PROFILE_MISMATCH for
 * refinement tables made for another descriptor or E or for other base
 * tables (their base id is not `tables`' profile id) and for a refinement
 * container made with other refinement tables, and KVC_ERR_CORRUPT_STREAM
 * for a refinement of another chunk (the token it was encoded from differs
 * from its base container's) or a damaged refinement stream.  Chunks are
 * grouped by level as in kvc_decode; each workgroup also stages the two
 * refinement models of every level it decodes.
 */
kvc_status kvc_decode_refined(const kvc_codec_desc *d, const void *tables, const void *rtables,
                              uint32_t refine_bits, const kvc_refined_chunk_ref *chunks,
                              uint32_t n_chunks, uint16_t *kv_out, uint32_t T_total, void *ws,
                              uint64_t ws_bytes, int32_t *dev_status, hipStream_t stream);

/* --------------------------------------------------------- streamed restore */
/*
 * Device staging bytes kvc_restore needs for these chunks in batches of
 * batch_chunks: three slots (fewer if there are fewer batches), each the
 * largest batch's containers, each container rounded up to 256 bytes.  0 for
 * an empty or invalid request.
 */
uint64_t kvc_restore_staging_bytes(const kvc_host_chunk *chunks, uint32_t n_chunks,
                                   uint32_t batch_chunks);

/*
 * Restore a context from containers in host memory, with the transfer of
 * one batch of chunks overlapping the decode of the one before (CacheGen
 * page, 核心方法, implementation paragraph: chunk i is sent while chunk i-1
 * is decoded).  chunks: host array of n_chunks, processed in order in
 * batches of batch_chunks (>= 1).  Batch b is copied host-to-device on
 * `copy` into staging slot b % 3 (device, staging_bytes >=
 * kvc_restore_staging_bytes), then decoded on `compute` exactly as
 * kvc_decode would decode those chunks (same kernels, same bits) into kv_out
 * [L][2][T_total][C]; the copy into a slot waits for the decode that last
 * read it, and the first copy waits for the work already queued on
 * `compute`.  ws: workspace of kvc_decode_ws_bytes(d, min(batch_chunks,
 * n_chunks)) bytes.  batch_done: NULL, or a host array of ceil(n_chunks /
 * batch_chunks) caller-created events, event b recorded on `compute` once
 * batch b is in kv_out.  All argument, range and size checks of every batch
 * are made before anything is queued.  On return everything is queued;
 * synchronizing `compute` waits for all of it.  `copy` and `compute` may be
 * the same stream (no overlap).  Device errors: those of kvc_decode, the
 * first one of any batch.
 */
kvc_status kvc_restore(const kvc_codec_desc *d, const void *tables, const kvc_host_chunk *chunks,
                       uint32_t n_chunks, uint32_t batch_chunks, uint16_t *kv_out,
                       uint32_t T_total, uint8_t *staging, uint64_t staging_bytes, void *ws,
                       uint64_t ws_bytes, int32_t *dev_status, hipStream_t compute,
                       hipStream_t copy, hipEvent_t *batch_done);

/* ---------------------------------------------------- per-chunk level choice */
/* One piece of a piecewise-constant bandwidth trace: from start_s (seconds,
 * increasing; the first is 0) until the next piece's start (the last piece
 * lasts forever) the link moves bytes_per_s (> 0) bytes per second. */
typedef struct {
  double start_s;
  double bytes_per_s;
} kvc_bw_piece;

/*
 * Per-chunk compression-level choice while streaming a context (CacheGen
 * page, 核心方法, online streaming paragraph: each chunk's level is chosen
 * from the previous chunk's measured throughput so that the remaining chunks
 * fit the TTFT SLO at the best quality; 关键观察, assumption 1: the estimate
 * lags by at most one chunk).  Host-only; simulates sending the chunks one
 * after another over `trace`, from time 0:
 *  - before chunk i the bandwidth estimate is init_bytes_per_s for i = 0,
 *    else chunk i-1's bytes / its transfer time (kept as it was if that
 *    time rounds to 0);
 *  - chunk i takes the lowest level index l (levels are ordered from best
 *    to worst quality) with  t + (sum over j >= i of chunk_bytes[j][l]) /
 *    estimate <= slo_s;  if no level fits, the level with the fewest
 *    remaining bytes (lowest index on a tie);
 *  - the chunk's bytes then move through the trace's pieces from time t.
 * chunk_bytes: host [n_chunks][n_levels] container sizes; levels_out: host
 * [n_chunks]; finish_s_out: host [n_chunks], each chunk's arrival time.  All
 * arithmetic is IEEE binary64 in the order written above.  Errors:
 * KVC_ERR_INVALID_ARG (null pointer, n_levels not in 1..255, a rate or the
 * estimate not positive and finite, pieces not starting at 0 or not
 * increasing, slo_s not finite).
 */
kvc_status kvc_plan_stream(const uint64_t *chunk_bytes, uint32_t n_chunks, uint32_t n_levels,
                           const kvc_bw_piece *trace, uint32_t n_pieces, double slo_s,
                           double init_bytes_per_s, uint8_t *levels_out, double *finish_s_out);

/*
 * Debug form of kvc_decode: same kernels, but writes the decoded symbols
 * (u8: anchor 0..255, delta q + M) to sym_out [L][2][T_total][C] instead of
 * binary16 values.
 */
kvc_status kvc_decode_symbols(const kvc_codec_desc *d, const void *tables,
                              const kvc_chunk_ref *chunks, uint32_t n_chunks, uint8_t *sym_out,
                              uint32_t T_total, void *ws, uint64_t ws_bytes, int32_t *dev_status,
                              hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* KVC_H_ */
