// Host side of the libkvc C ABI: argument validation, workspace layout and
// the stream-ordered launch sequences of profile / encode / decode.
#include <algorithm>
#include <vector>

#include "kvc_internal.h"

namespace kvc {
hipError_t launch_reset_status(int32_t *status, hipStream_t stream);
hipError_t launch_load_chunks(const ChunkInfo *host_chunks, uint32_t n_chunks,
                              ChunkInfo *dev_chunks, uint32_t *flags, hipStream_t stream);
hipError_t launch_index(const Desc &d, const ChunkInfo *dev_chunks, uint32_t n_chunks,
                        uint64_t *row_sums, uint32_t *flags, uint32_t *offsets, uint8_t *valid,
                        uint64_t *payload, const uint8_t *tables, int check_header_flag,
                        int32_t *status, hipStream_t stream);
hipError_t launch_load_groups(const DecodeGroup *host_groups, uint32_t n_groups,
                              DecodeGroup *dev_groups, hipStream_t stream);
hipError_t launch_decode(const Desc &d, const ChunkInfo *dev_chunks, const DecodeGroup *groups,
                         uint32_t n_groups, uint32_t levels, uint32_t waves, const uint8_t *valid,
                         const uint32_t *offsets, const uint8_t *tables, bool symbols,
                         int32_t *status, hipStream_t stream);
size_t decode_lds_bytes(uint32_t levels, uint32_t waves);
hipError_t launch_encode(const Desc &d, const uint8_t *tables, const uint16_t *kv, uint32_t T,
                         const ChunkInfo *dev_chunks, uint32_t n_chunks,
                         const DecodeGroup *groups, uint32_t n_groups, uint32_t levels,
                         uint32_t waves, uint8_t *records, uint64_t *row_sums, uint32_t *flags,
                         uint32_t *offsets, uint8_t *valid, uint64_t *payload,
                         uint64_t *chunk_off_ws, uint32_t *fits, uint32_t *redo,
                         uint8_t *redo_scratch, uint32_t redo_blocks, uint8_t *out,
                         uint64_t out_cap, uint64_t *chunk_off_out, int32_t *status,
                         hipStream_t stream);
uint32_t encode_redo_lane_bytes(uint32_t chunk);
size_t encode_lds_bytes(uint32_t levels);
size_t encode_emit_lds_bytes(uint32_t levels, uint32_t waves);
hipError_t launch_profile(const Desc &d, const uint16_t *kv, uint32_t T, uint8_t *tables,
                          uint32_t *counts, uint64_t *model_hash, uint64_t *row_hash,
                          int32_t *status, hipStream_t stream);
hipError_t launch_profile_refine(const Desc &d, uint32_t ebits, const uint16_t *kv, uint32_t T,
                                 const uint8_t *base_tables, uint8_t *rtables, uint32_t *counts,
                                 uint64_t *model_hash, uint64_t *row_hash, int32_t *status,
                                 hipStream_t stream);
size_t refine_count_lds_bytes(const Desc &d);
uint32_t refine_emit_lane_bytes(uint32_t chunk);
hipError_t launch_encode_refine(const Desc &d, uint32_t ebits, const uint8_t *rtables,
                                const uint16_t *kv, uint32_t T, const ChunkInfo *dev_chunks,
                                uint32_t n_chunks, uint32_t stat_blocks, uint32_t emit_blocks,
                                float *side, uint8_t *records, uint64_t *row_sums,
                                uint32_t *flags, uint32_t *offsets, uint8_t *valid,
                                uint64_t *payload, uint64_t *chunk_off_ws, uint32_t *fits,
                                uint32_t *spare, uint8_t *scratch, uint8_t *out, uint64_t out_cap,
                                uint64_t *chunk_off_out, int32_t *status, hipStream_t stream);
size_t decode_refined_lds_bytes(uint32_t levels, uint32_t ebits, uint32_t waves);
hipError_t launch_decode_refined(const Desc &d, uint32_t ebits, const ChunkInfo *dev_chunks,
                                 const ChunkInfo *dev_rchunks, const DecodeGroup *groups,
                                 uint32_t n_groups, uint32_t levels, uint32_t waves,
                                 const uint8_t *valid,
                                 const uint8_t *rvalid, const uint32_t *offsets,
                                 const uint32_t *roffsets, const uint8_t *tables,
                                 const uint8_t *rtables, int32_t *status, hipStream_t stream);
}  // namespace kvc

using namespace kvc;

namespace {

bool desc_ok(const kvc_codec_desc *d) {
  if (!d) return false;
  if (d->n_layers < 1 || d->n_layers > 32767) return false;
  if (d->n_channels < 1 || d->n_channels > (1u << 24)) return false;
  if ((uint64_t)2 * d->n_layers * d->n_channels >= (1ull << 31)) return false;
  if (d->chunk_tokens < 1 || d->chunk_tokens > 65535) return false;
  if (d->group_tokens < 1 || d->group_tokens > d->chunk_tokens) return false;
  if (d->anchor_bits != 8 || d->cdf_prec_bits != kPrec) return false;
  if (d->n_levels < 1 || d->n_levels > 4) return false;
  for (uint32_t lv = 0; lv < d->n_levels; ++lv)
    for (int t = 0; t < 3; ++t)
      if (d->delta_bits[lv][t] < 2 || d->delta_bits[lv][t] > 6) return false;
  return true;
}

Desc to_desc(const kvc_codec_desc *d) {
  Desc r;
  r.L = d->n_layers;
  r.C = d->n_channels;
  r.G = d->group_tokens;
  r.chunk = d->chunk_tokens;
  r.nlev = d->n_levels;
  for (int lv = 0; lv < 4; ++lv)
    for (int t = 0; t < 3; ++t) r.bits[lv][t] = lv < (int)d->n_levels ? d->delta_bits[lv][t] : 0;
  return r;
}

bool aligned(const void *p, uintptr_t a) { return ((uintptr_t)p % a) == 0; }

// Workgroups (one wave each) of the encoder's slow path, and the scratch
// they share: at most 8, fewer when a chunk's scratch is large.
uint32_t redo_blocks(const Desc &d) {
  const uint64_t per = (uint64_t)kWave * encode_redo_lane_bytes(d.chunk);
  return (uint32_t)std::max<uint64_t>(1, std::min<uint64_t>(8, (16ull << 20) / per));
}

// Workspace layout shared by decode and encode (encode adds its tail).
struct WsLayout {
  uint64_t chunks, groups, rows, hdr, valid, payload, offsets, records, chunk_off, fits, redo,
      redo_scratch, total;
};

WsLayout ws_layout(const Desc &d, uint32_t K, bool encode) {
  const uint64_t S = n_streams(d);
  WsLayout w;
  w.chunks = 0;
  w.groups = align256(w.chunks + (uint64_t)K * sizeof(ChunkInfo));
  w.rows = align256(w.groups + (uint64_t)K * sizeof(DecodeGroup));
  w.hdr = align256(w.rows + (uint64_t)K * 2 * d.L * 8);
  w.valid = align256(w.hdr + (uint64_t)K * 4);
  w.payload = align256(w.valid + K);
  w.offsets = align256(w.payload + (uint64_t)K * 8);
  uint64_t end = w.offsets + (uint64_t)K * S * 4;
  w.records = w.chunk_off = w.fits = w.redo = w.redo_scratch = 0;
  if (encode) {
    // the slow path's list: a count, then (chunk, unit) pairs, at most one
    // per chunk and unit
    const uint64_t units = 2ull * d.L * ((d.C + kWave - 1) / kWave);
    w.records = align256(end);
    w.chunk_off = align256(w.records + (uint64_t)K * S * kRecBytes);
    w.fits = align256(w.chunk_off + (uint64_t)(K + 1) * 8);
    w.redo = align256(w.fits + 4);
    w.redo_scratch = align256(w.redo + 4 + 8 * (uint64_t)K * units);
    end = w.redo_scratch + (uint64_t)redo_blocks(d) * kWave * encode_redo_lane_bytes(d.chunk);
  }
  w.total = align256(end);
  return w;
}

uint64_t container_bound_n(const Desc &d, uint32_t n) {
  const uint64_t S = n_streams(d);
  return kHdrBytes + kRecBytes * S + S * pad8(4ull + 2ull * n);
}

kvc_status hip_status(hipError_t e) { return e == hipSuccess ? KVC_OK : KVC_ERR_HIP; }

// A chunk to decode and the output cache its values go to.
struct OutChunk {
  kvc_chunk_ref r;
  void *out;   // [L][2][T][C] binary16 (values) or u8 (symbols)
  uint32_t T;  // that cache's token capacity
};

kvc_status decode_chunks(const kvc_codec_desc *dd, const void *tables, const OutChunk *chunks,
                         uint32_t n_chunks, void *ws, uint64_t ws_bytes, int32_t *dev_status,
                         hipStream_t stream, int mode, uint32_t *offsets_out,
                         bool reset_status = true) {
  // mode 0: values, 1: symbols, 2: index only
  if (!desc_ok(dd)) return KVC_ERR_INVALID_ARG;
  const Desc d = to_desc(dd);
  if (!tables || !aligned(tables, 16) || !dev_status || !aligned(dev_status, 4))
    return KVC_ERR_INVALID_ARG;
  if (n_chunks > 65535) return KVC_ERR_SHAPE;
  if (n_chunks && !chunks) return KVC_ERR_INVALID_ARG;
  const uint32_t esz = mode == 0 ? 2 : 1;
  for (uint32_t k = 0; mode != 2 && k < n_chunks; ++k)
    if (!chunks[k].out || !aligned(chunks[k].out, esz)) return KVC_ERR_INVALID_ARG;
  if (mode == 2 && n_chunks && (!offsets_out || !aligned(offsets_out, 4)))
    return KVC_ERR_INVALID_ARG;
  const WsLayout w = ws_layout(d, n_chunks, false);
  if (n_chunks && (!ws || !aligned(ws, 256))) return KVC_ERR_INVALID_ARG;
  if (ws_bytes < w.total) return KVC_ERR_CAPACITY;
  const uint64_t S = n_streams(d);
  std::vector<ChunkInfo> info(n_chunks);
  struct Range {
    uintptr_t out;
    uint32_t T, a, b;
  };
  std::vector<Range> ranges(n_chunks);
  for (uint32_t k = 0; k < n_chunks; ++k) {
    const kvc_chunk_ref &c = chunks[k].r;
    if (!c.container || !aligned(c.container, 4)) return KVC_ERR_INVALID_ARG;
    if (c.level >= d.nlev || c.reserved != 0) return KVC_ERR_INVALID_ARG;
    if (c.n_tokens < 1 || c.n_tokens > d.chunk) return KVC_ERR_SHAPE;
    if (mode != 2 && (uint64_t)c.first_token + c.n_tokens > chunks[k].T) return KVC_ERR_SHAPE;
    if (c.container_bytes < kHdrBytes + kRecBytes * S) return KVC_ERR_SHAPE;
    // decode reads containers through 32-bit bounded buffer resources
    if (c.container_bytes > 0xFFFFFFFFull) return KVC_ERR_SHAPE;
    info[k].cont = c.container;
    info[k].records = c.container + kHdrBytes;
    info[k].cont_bytes = c.container_bytes;
    info[k].first_token = c.first_token;
    info[k].n_tokens = c.n_tokens;
    info[k].level = c.level;
    info[k].out_tokens = mode == 2 ? 0 : chunks[k].T;
    info[k].out = mode == 2 ? nullptr : chunks[k].out;
    ranges[k] = {(uintptr_t)chunks[k].out, chunks[k].T, c.first_token, c.first_token + c.n_tokens};
  }
  if (mode != 2 && n_chunks) {
    // chunks sharing an output cache: one token capacity, disjoint token
    // ranges; distinct output caches must not overlap in memory
    std::sort(ranges.begin(), ranges.end(), [](const Range &x, const Range &y) {
      return x.out != y.out ? x.out < y.out : x.a < y.a;
    });
    const uint64_t row_bytes = 2ull * d.L * d.C * esz;  // [L][2] rows of C per token
    for (uint32_t k = 1; k < n_chunks; ++k) {
      const Range &p = ranges[k - 1], &q = ranges[k];
      if (q.out == p.out) {
        if (q.T != p.T || q.a < p.b) return KVC_ERR_SHAPE;
      } else if (q.out < p.out + row_bytes * p.T) {
        return KVC_ERR_SHAPE;
      }
    }
  }
  // Decode groups (values / symbols): the chunk table is ordered by level so
  // that a group's chunks span few levels (fewer delta models to stage),
  // then split into near-equal groups, each decoded by one workgroup per
  // (row, channel block) whose waves take at most kMaxRounds chunks each.
  // The index-only call keeps the caller's order.
  std::vector<DecodeGroup> groups;
  uint32_t levels = 1, waves = 1;
  if (mode != 2 && n_chunks) {
    std::stable_sort(info.begin(), info.end(),
                     [](const ChunkInfo &a, const ChunkInfo &b) { return a.level < b.level; });
    constexpr uint32_t kMaxRounds = 4;
    uint32_t all_levels = 0;
    for (const ChunkInfo &c : info) all_levels |= 1u << c.level;
    const uint32_t lv_all = (uint32_t)__builtin_popcount(all_levels);
    uint32_t wmax = 1;
    for (uint32_t w = kDecodeMaxWaves; w >= 1; --w)
      if (decode_lds_bytes(lv_all, w) <= kLdsBudget) {
        wmax = w;
        break;
      }
    const uint32_t ng = (n_chunks + wmax * kMaxRounds - 1) / (wmax * kMaxRounds);
    for (uint32_t gi = 0; gi < ng; ++gi) {
      const uint32_t a = (uint32_t)((uint64_t)n_chunks * gi / ng);
      const uint32_t b = (uint32_t)((uint64_t)n_chunks * (gi + 1) / ng);
      DecodeGroup g{};
      g.start = a;
      g.count = b - a;
      for (uint32_t i = a; i < b; ++i) g.level |= 1u << info[i].level;
      levels = std::max<uint32_t>(levels, (uint32_t)__builtin_popcount(g.level));
      waves = std::max<uint32_t>(waves, std::min<uint32_t>(wmax, g.count));
      groups.push_back(g);
    }
  }
  hipError_t e = reset_status ? launch_reset_status(dev_status, stream) : hipSuccess;
  if (e != hipSuccess || n_chunks == 0) return hip_status(e);
  uint8_t *base = static_cast<uint8_t *>(ws);
  ChunkInfo *dch = reinterpret_cast<ChunkInfo *>(base + w.chunks);
  uint32_t *offs = mode == 2 ? offsets_out : reinterpret_cast<uint32_t *>(base + w.offsets);
  e = launch_load_chunks(info.data(), n_chunks, dch, reinterpret_cast<uint32_t *>(base + w.hdr),
                         stream);
  if (e != hipSuccess) return KVC_ERR_HIP;
  e = launch_index(d, dch, n_chunks, reinterpret_cast<uint64_t *>(base + w.rows),
                   reinterpret_cast<uint32_t *>(base + w.hdr),
                   offs, base + w.valid, reinterpret_cast<uint64_t *>(base + w.payload),
                   static_cast<const uint8_t *>(tables), 1, dev_status, stream);
  if (e != hipSuccess || mode == 2) return hip_status(e);
  DecodeGroup *dgr = reinterpret_cast<DecodeGroup *>(base + w.groups);
  e = launch_load_groups(groups.data(), (uint32_t)groups.size(), dgr, stream);
  if (e != hipSuccess) return KVC_ERR_HIP;
  e = launch_decode(d, dch, dgr, (uint32_t)groups.size(), levels, waves, base + w.valid, offs,
                    static_cast<const uint8_t *>(tables), mode == 1, dev_status, stream);
  return hip_status(e);
}

// Every chunk into one output cache.
kvc_status decode_common(const kvc_codec_desc *dd, const void *tables, const kvc_chunk_ref *chunks,
                         uint32_t n_chunks, void *out, uint32_t T_total, void *ws,
                         uint64_t ws_bytes, int32_t *dev_status, hipStream_t stream, int mode,
                         uint32_t *offsets_out, bool reset_status = true) {
  if (n_chunks && !chunks) return KVC_ERR_INVALID_ARG;
  if (n_chunks > 65535) return KVC_ERR_SHAPE;
  std::vector<OutChunk> v(n_chunks);
  for (uint32_t k = 0; k < n_chunks; ++k) v[k] = {chunks[k], out, T_total};
  return decode_chunks(dd, tables, v.data(), n_chunks, ws, ws_bytes, dev_status, stream, mode,
                       offsets_out, reset_status);
}

// Largest batch of a restore: the sum of its containers, each rounded up to
// 256 bytes (the staging slot size).
uint64_t restore_slot_bytes(const kvc_host_chunk *c, uint32_t n, uint32_t batch) {
  uint64_t best = 0;
  for (uint32_t b0 = 0; b0 < n; b0 += batch) {
    uint64_t sum = 0;
    for (uint32_t k = b0; k < n && k - b0 < batch; ++k) sum += align256(c[k].container_bytes);
    best = std::max(best, sum);
  }
  return best;
}

// Staging slots of a restore: a batch's copy waits only for the decode of
// the batch kRestoreSlots earlier, so copies run ahead of slow decodes.
constexpr uint32_t kRestoreSlots = 3;

// Events of one restore call, destroyed when the call returns (a recorded
// event may be destroyed before it completes; the runtime releases it then).
struct RestoreEvents {
  hipEvent_t ev[2 * kRestoreSlots + 1] = {};
  hipError_t create() {
    for (hipEvent_t &e : ev) {
      const hipError_t r = hipEventCreateWithFlags(&e, hipEventDisableTiming);
      if (r != hipSuccess) return r;
    }
    return hipSuccess;
  }
  ~RestoreEvents() {
    for (hipEvent_t e : ev)
      if (e) (void)hipEventDestroy(e);
  }
};

// ---------------------------------------------------------- refinement
constexpr uint32_t kRefineMinBits = 2, kRefineMaxBits = 6;
bool refine_bits_ok(uint32_t e) { return e >= kRefineMinBits && e <= kRefineMaxBits; }

// Refinement encode: one wave per (chunk, unit) item; the emit waves share
// at most this much scratch (about 14 waves per CU at 1,500-token chunks).
constexpr uint64_t kRefineScratchCap = 1ull << 30;
uint32_t refine_items(const Desc &d, uint32_t K) {
  return K * 2u * d.L * ((d.C + kWave - 1) / kWave);
}
uint32_t refine_emit_blocks(const Desc &d, uint32_t K) {
  const uint64_t per = (uint64_t)kWave * refine_emit_lane_bytes(d.chunk);
  const uint64_t cap = std::max<uint64_t>(1, kRefineScratchCap / per);
  return (uint32_t)std::max<uint64_t>(1, std::min<uint64_t>({cap, 4096, refine_items(d, K)}));
}
uint32_t refine_stat_blocks(const Desc &d, uint32_t K) {
  return std::max<uint32_t>(1, std::min<uint32_t>(4096, refine_items(d, K)));
}

struct RefineEncodeWs {
  uint64_t chunks, rows, hdr, valid, payload, offsets, records, side, chunk_off, fits, spare,
      scratch, total;
};
RefineEncodeWs refine_encode_ws(const Desc &d, uint32_t K) {
  const uint64_t S = n_streams(d);
  RefineEncodeWs w;
  w.chunks = 0;
  w.rows = align256((uint64_t)K * sizeof(ChunkInfo));
  w.hdr = align256(w.rows + (uint64_t)K * 2 * d.L * 8);
  w.valid = align256(w.hdr + (uint64_t)K * 4);
  w.payload = align256(w.valid + K);
  w.offsets = align256(w.payload + (uint64_t)K * 8);
  w.records = align256(w.offsets + (uint64_t)K * S * 4);
  w.side = align256(w.records + (uint64_t)K * S * kRecBytes);
  w.chunk_off = align256(w.side + (uint64_t)K * S * 16);
  w.fits = align256(w.chunk_off + (uint64_t)(K + 1) * 8);
  w.spare = align256(w.fits + 4);
  w.scratch = align256(w.spare + 4);
  w.total = align256(w.scratch + (uint64_t)refine_emit_blocks(d, K) * kWave *
                                     refine_emit_lane_bytes(d.chunk));
  return w;
}

}  // namespace

extern "C" {

int kvc_version(void) { return 100; }

const char *kvc_status_str(kvc_status s) {
  switch (s) {
    case KVC_OK: return "ok";
    case KVC_ERR_INVALID_ARG: return "invalid argument";
    case KVC_ERR_SHAPE: return "inconsistent shape or token range";
    case KVC_ERR_PROFILE_MISMATCH: return "container was encoded with other tables";
    case KVC_ERR_CORRUPT_STREAM: return "corrupt container or bitstream";
    case KVC_ERR_NONFINITE: return "non-finite value in the input";
    case KVC_ERR_CAPACITY: return "buffer or workspace too small";
    case KVC_ERR_HIP: return "HIP runtime error";
    case KVC_ERR_UNIMPLEMENTED: return "not implemented";
  }
  return "unknown status";
}

kvc_status kvc_validate_desc(const kvc_codec_desc *d) {
  return desc_ok(d) ? KVC_OK : KVC_ERR_INVALID_ARG;
}

uint64_t kvc_tables_bytes(const kvc_codec_desc *dd) {
  if (!desc_ok(dd)) return 0;
  const uint64_t S = 2ull * dd->n_layers * dd->n_channels;
  return kTablesHdr + S * kAnchorStride * 2 + (uint64_t)dd->n_levels * S * kDeltaStride * 2;
}

uint64_t kvc_profile_ws_bytes(const kvc_codec_desc *dd) {
  if (!desc_ok(dd)) return 0;
  const uint64_t S = 2ull * dd->n_layers * dd->n_channels;
  const uint64_t counts = S * (kAnchorAlpha + (uint64_t)dd->n_levels * kDeltaStride) * 4;
  return align256(counts) + align256(S * 8) + align256(2ull * dd->n_layers * 8);
}

kvc_status kvc_profile(const kvc_codec_desc *dd, const uint16_t *kv_fp16, uint32_t T,
                       void *tables_out, void *ws, uint64_t ws_bytes, int32_t *dev_status,
                       hipStream_t stream) {
  if (!desc_ok(dd)) return KVC_ERR_INVALID_ARG;
  if (!kv_fp16 || !aligned(kv_fp16, 2) || !tables_out || !aligned(tables_out, 16) || !ws ||
      !aligned(ws, 256) || !dev_status || !aligned(dev_status, 4))
    return KVC_ERR_INVALID_ARG;
  if (T < 1) return KVC_ERR_SHAPE;
  if (ws_bytes < kvc_profile_ws_bytes(dd)) return KVC_ERR_CAPACITY;
  const Desc d = to_desc(dd);
  const uint64_t S = n_streams(d);
  uint8_t *base = static_cast<uint8_t *>(ws);
  const uint64_t counts_bytes = S * (kAnchorAlpha + (uint64_t)d.nlev * kDeltaStride) * 4;
  uint32_t *counts = reinterpret_cast<uint32_t *>(base);
  uint64_t *model_hash = reinterpret_cast<uint64_t *>(base + align256(counts_bytes));
  uint64_t *row_hash = reinterpret_cast<uint64_t *>(base + align256(counts_bytes) + align256(S * 8));
  hipError_t e = launch_reset_status(dev_status, stream);
  if (e != hipSuccess) return KVC_ERR_HIP;
  e = launch_profile(d, kv_fp16, T, static_cast<uint8_t *>(tables_out), counts, model_hash,
                     row_hash, dev_status, stream);
  return hip_status(e);
}

uint64_t kvc_container_bound(const kvc_codec_desc *dd, uint32_t n_tokens) {
  if (!desc_ok(dd)) return 0;
  return container_bound_n(to_desc(dd), n_tokens);
}

uint64_t kvc_encode_bound(const kvc_codec_desc *dd, uint32_t T) {
  if (!desc_ok(dd)) return 0;
  const Desc d = to_desc(dd);
  uint64_t total = 0;
  for (uint64_t t0 = 0; t0 < T; t0 += d.chunk)
    total += container_bound_n(d, (uint32_t)std::min<uint64_t>(d.chunk, T - t0));
  return total;
}

uint64_t kvc_encode_ws_bytes(const kvc_codec_desc *dd, uint32_t T) {
  if (!desc_ok(dd)) return 0;
  const Desc d = to_desc(dd);
  const uint32_t K = (uint32_t)((T + (uint64_t)d.chunk - 1) / d.chunk);
  return ws_layout(d, K, true).total;
}

kvc_status kvc_encode(const kvc_codec_desc *dd, const void *tables, const uint16_t *kv_fp16,
                      uint32_t T, const uint8_t *chunk_levels, uint8_t *out, uint64_t out_cap,
                      uint64_t *chunk_offsets_out, void *ws, uint64_t ws_bytes,
                      int32_t *dev_status, hipStream_t stream) {
  if (!desc_ok(dd)) return KVC_ERR_INVALID_ARG;
  const Desc d = to_desc(dd);
  if (!tables || !aligned(tables, 16) || !kv_fp16 || !aligned(kv_fp16, 2) || !chunk_levels ||
      !out || !aligned(out, 4) || !chunk_offsets_out || !aligned(chunk_offsets_out, 8) || !ws ||
      !aligned(ws, 256) || !dev_status || !aligned(dev_status, 4))
    return KVC_ERR_INVALID_ARG;
  if (T < 1) return KVC_ERR_SHAPE;
  const uint64_t K64 = (T + (uint64_t)d.chunk - 1) / d.chunk;
  if (K64 > 65535) return KVC_ERR_SHAPE;
  const uint32_t K = (uint32_t)K64;
  const uint64_t S = n_streams(d);
  // every stream offset inside a chunk's payload is a u32
  if (S * pad8(4ull + 2ull * d.chunk) > 0xFFFFFFFFull) return KVC_ERR_SHAPE;
  const WsLayout w = ws_layout(d, K, true);
  if (ws_bytes < w.total) return KVC_ERR_CAPACITY;
  uint8_t *base = static_cast<uint8_t *>(ws);
  std::vector<ChunkInfo> info(K);
  for (uint32_t k = 0; k < K; ++k) {
    if (chunk_levels[k] >= d.nlev) return KVC_ERR_INVALID_ARG;
    const uint64_t t0 = (uint64_t)k * d.chunk;
    info[k].cont = nullptr;
    info[k].records = base + w.records + (uint64_t)k * S * kRecBytes;
    info[k].cont_bytes = 0;
    info[k].first_token = (uint32_t)t0;
    info[k].n_tokens = (uint32_t)std::min<uint64_t>(d.chunk, T - t0);
    info[k].level = chunk_levels[k];
    info[k].out_tokens = 0;
    info[k].out = nullptr;
  }
  hipError_t e = launch_reset_status(dev_status, stream);
  if (e != hipSuccess) return KVC_ERR_HIP;
  ChunkInfo *dch = reinterpret_cast<ChunkInfo *>(base + w.chunks);
  e = launch_load_chunks(info.data(), K, dch, reinterpret_cast<uint32_t *>(base + w.hdr), stream);
  if (e != hipSuccess) return KVC_ERR_HIP;
  // Encode groups: contiguous chunk ranges, each encoded by one workgroup
  // per (row, channel block) that stages the models of the levels it uses;
  // its waves take the group's chunks in turn, at most kMaxRounds each.  A
  // workgroup has as many waves as the group has chunks, up to the most
  // whose models and block queues still let two emit workgroups share a CU.
  std::vector<DecodeGroup> groups;
  uint32_t levels = 1, waves = 1;
  {
    constexpr uint32_t kMaxRounds = 4;
    uint32_t all_levels = 0;
    for (uint32_t k = 0; k < K; ++k) all_levels |= 1u << chunk_levels[k];
    const uint32_t lv_all = (uint32_t)__builtin_popcount(all_levels);
    uint32_t wmax = 1;
    for (uint32_t w = kEncodeMaxWaves; w >= 1; --w)
      if (encode_emit_lds_bytes(lv_all, w) <= kLdsBudget) {
        wmax = w;
        break;
      }
    const uint32_t per = wmax * kMaxRounds;
    const uint32_t ng = (K + per - 1) / per;
    for (uint32_t gi = 0; gi < ng; ++gi) {
      const uint32_t a = (uint32_t)((uint64_t)K * gi / ng);
      const uint32_t b = (uint32_t)((uint64_t)K * (gi + 1) / ng);
      DecodeGroup g{};
      g.start = a;
      g.count = b - a;
      for (uint32_t i = a; i < b; ++i) g.level |= 1u << chunk_levels[i];
      levels = std::max<uint32_t>(levels, (uint32_t)__builtin_popcount(g.level));
      waves = std::max<uint32_t>(waves, std::min<uint32_t>(wmax, g.count));
      groups.push_back(g);
    }
  }
  DecodeGroup *dgr = reinterpret_cast<DecodeGroup *>(base + w.groups);
  e = launch_load_groups(groups.data(), (uint32_t)groups.size(), dgr, stream);
  if (e != hipSuccess) return KVC_ERR_HIP;
  e = launch_encode(d, static_cast<const uint8_t *>(tables), kv_fp16, T, dch, K, dgr,
                    (uint32_t)groups.size(), levels, waves, base + w.records,
                    reinterpret_cast<uint64_t *>(base + w.rows),
                    reinterpret_cast<uint32_t *>(base + w.hdr),
                    reinterpret_cast<uint32_t *>(base + w.offsets), base + w.valid,
                    reinterpret_cast<uint64_t *>(base + w.payload),
                    reinterpret_cast<uint64_t *>(base + w.chunk_off),
                    reinterpret_cast<uint32_t *>(base + w.fits),
                    reinterpret_cast<uint32_t *>(base + w.redo), base + w.redo_scratch,
                    redo_blocks(d), out, out_cap, chunk_offsets_out, dev_status, stream);
  return hip_status(e);
}

uint64_t kvc_decode_ws_bytes(const kvc_codec_desc *dd, uint32_t n_chunks) {
  if (!desc_ok(dd)) return 0;
  return ws_layout(to_desc(dd), n_chunks, false).total;
}

kvc_status kvc_decode(const kvc_codec_desc *d, const void *tables, const kvc_chunk_ref *chunks,
                      uint32_t n_chunks, uint16_t *kv_out, uint32_t T_total, void *ws,
                      uint64_t ws_bytes, int32_t *dev_status, hipStream_t stream) {
  return decode_common(d, tables, chunks, n_chunks, kv_out, T_total, ws, ws_bytes, dev_status,
                       stream, 0, nullptr);
}

kvc_status kvc_decode_symbols(const kvc_codec_desc *d, const void *tables,
                              const kvc_chunk_ref *chunks, uint32_t n_chunks, uint8_t *sym_out,
                              uint32_t T_total, void *ws, uint64_t ws_bytes, int32_t *dev_status,
                              hipStream_t stream) {
  return decode_common(d, tables, chunks, n_chunks, sym_out, T_total, ws, ws_bytes, dev_status,
                       stream, 1, nullptr);
}

kvc_status kvc_decode_index(const kvc_codec_desc *d, const void *tables,
                            const kvc_chunk_ref *chunks, uint32_t n_chunks, uint32_t *offsets_out,
                            void *ws, uint64_t ws_bytes, int32_t *dev_status, hipStream_t stream) {
  return decode_common(d, tables, chunks, n_chunks, nullptr, 0, ws, ws_bytes, dev_status, stream,
                       2, offsets_out);
}

kvc_status kvc_decode_multi(const kvc_codec_desc *d, const void *tables,
                            const kvc_request_chunk *chunks, uint32_t n_chunks, void *ws,
                            uint64_t ws_bytes, int32_t *dev_status, hipStream_t stream) {
  if (n_chunks && !chunks) return KVC_ERR_INVALID_ARG;
  if (n_chunks > 65535) return KVC_ERR_SHAPE;
  std::vector<OutChunk> v(n_chunks);
  for (uint32_t k = 0; k < n_chunks; ++k) {
    const kvc_request_chunk &c = chunks[k];
    if (c.reserved2 != 0) return KVC_ERR_INVALID_ARG;
    v[k] = {{c.container, c.container_bytes, c.first_token, c.n_tokens, c.level, c.reserved},
            c.kv_out, c.T_total};
  }
  return decode_chunks(d, tables, v.data(), n_chunks, ws, ws_bytes, dev_status, stream, 0,
                       nullptr);
}

// ---------------------------------------------------------- refinement
uint64_t kvc_refine_tables_bytes(const kvc_codec_desc *dd) {
  if (!desc_ok(dd)) return 0;
  const uint64_t S = 2ull * dd->n_layers * dd->n_channels;
  return kTablesHdr + 2ull * dd->n_levels * S * kDeltaStride * 2;
}

uint64_t kvc_refine_profile_ws_bytes(const kvc_codec_desc *dd) {
  if (!desc_ok(dd)) return 0;
  const uint64_t S = 2ull * dd->n_layers * dd->n_channels;
  const uint64_t counts = S * 2ull * dd->n_levels * kDeltaStride * 4;
  return align256(counts) + align256(S * 8) + align256(2ull * dd->n_layers * 8);
}

kvc_status kvc_profile_refine(const kvc_codec_desc *dd, const void *tables,
                              const uint16_t *kv_fp16, uint32_t T, uint32_t refine_bits,
                              void *rtables_out, void *ws, uint64_t ws_bytes, int32_t *dev_status,
                              hipStream_t stream) {
  if (!desc_ok(dd) || !refine_bits_ok(refine_bits)) return KVC_ERR_INVALID_ARG;
  if (!tables || !aligned(tables, 16) || !kv_fp16 || !aligned(kv_fp16, 2) || !rtables_out ||
      !aligned(rtables_out, 16) || !ws || !aligned(ws, 256) || !dev_status ||
      !aligned(dev_status, 4))
    return KVC_ERR_INVALID_ARG;
  if (T < 1) return KVC_ERR_SHAPE;
  if (ws_bytes < kvc_refine_profile_ws_bytes(dd)) return KVC_ERR_CAPACITY;
  const Desc d = to_desc(dd);
  const uint64_t S = n_streams(d);
  if (refine_count_lds_bytes(d) > 64 * 1024) return KVC_ERR_INVALID_ARG;
  uint8_t *base = static_cast<uint8_t *>(ws);
  const uint64_t counts_bytes = S * 2ull * d.nlev * kDeltaStride * 4;
  uint32_t *counts = reinterpret_cast<uint32_t *>(base);
  uint64_t *model_hash = reinterpret_cast<uint64_t *>(base + align256(counts_bytes));
  uint64_t *row_hash = reinterpret_cast<uint64_t *>(base + align256(counts_bytes) + align256(S * 8));
  hipError_t e = launch_reset_status(dev_status, stream);
  if (e != hipSuccess) return KVC_ERR_HIP;
  e = launch_profile_refine(d, refine_bits, kv_fp16, T, static_cast<const uint8_t *>(tables),
                            static_cast<uint8_t *>(rtables_out), counts, model_hash, row_hash,
                            dev_status, stream);
  return hip_status(e);
}

uint64_t kvc_encode_refine_ws_bytes(const kvc_codec_desc *dd, uint32_t T) {
  if (!desc_ok(dd)) return 0;
  const Desc d = to_desc(dd);
  const uint32_t K = (uint32_t)((T + (uint64_t)d.chunk - 1) / d.chunk);
  return refine_encode_ws(d, K).total;
}

kvc_status kvc_encode_refine(const kvc_codec_desc *dd, const void *rtables, uint32_t refine_bits,
                             const uint16_t *kv_fp16, uint32_t T, const uint8_t *chunk_levels,
                             uint8_t *out, uint64_t out_cap, uint64_t *chunk_offsets_out,
                             void *ws, uint64_t ws_bytes, int32_t *dev_status,
                             hipStream_t stream) {
  if (!desc_ok(dd) || !refine_bits_ok(refine_bits)) return KVC_ERR_INVALID_ARG;
  const Desc d = to_desc(dd);
  if (!rtables || !aligned(rtables, 16) || !kv_fp16 || !aligned(kv_fp16, 2) || !chunk_levels ||
      !out || !aligned(out, 4) || !chunk_offsets_out || !aligned(chunk_offsets_out, 8) || !ws ||
      !aligned(ws, 256) || !dev_status || !aligned(dev_status, 4))
    return KVC_ERR_INVALID_ARG;
  if (T < 1) return KVC_ERR_SHAPE;
  const uint64_t K64 = (T + (uint64_t)d.chunk - 1) / d.chunk;
  if (K64 > 65535) return KVC_ERR_SHAPE;
  const uint32_t K = (uint32_t)K64;
  const uint64_t S = n_streams(d);
  if (S * pad8(4ull + 2ull * d.chunk) > 0xFFFFFFFFull) return KVC_ERR_SHAPE;
  const RefineEncodeWs w = refine_encode_ws(d, K);
  if (ws_bytes < w.total) return KVC_ERR_CAPACITY;
  uint8_t *base = static_cast<uint8_t *>(ws);
  std::vector<ChunkInfo> info(K);
  for (uint32_t k = 0; k < K; ++k) {
    if (chunk_levels[k] >= d.nlev) return KVC_ERR_INVALID_ARG;
    const uint64_t t0 = (uint64_t)k * d.chunk;
    info[k].cont = nullptr;
    info[k].records = base + w.records + (uint64_t)k * S * kRecBytes;
    info[k].cont_bytes = 0;
    info[k].first_token = (uint32_t)t0;
    info[k].n_tokens = (uint32_t)std::min<uint64_t>(d.chunk, T - t0);
    info[k].level = chunk_levels[k];
    info[k].out_tokens = 0;
    info[k].out = nullptr;
  }
  hipError_t e = launch_reset_status(dev_status, stream);
  if (e != hipSuccess) return KVC_ERR_HIP;
  ChunkInfo *dch = reinterpret_cast<ChunkInfo *>(base + w.chunks);
  e = launch_load_chunks(info.data(), K, dch, reinterpret_cast<uint32_t *>(base + w.hdr), stream);
  if (e != hipSuccess) return KVC_ERR_HIP;
  e = launch_encode_refine(d, refine_bits, static_cast<const uint8_t *>(rtables), kv_fp16, T, dch,
                           K, refine_stat_blocks(d, K), refine_emit_blocks(d, K),
                           reinterpret_cast<float *>(base + w.side), base + w.records,
                           reinterpret_cast<uint64_t *>(base + w.rows),
                           reinterpret_cast<uint32_t *>(base + w.hdr),
                           reinterpret_cast<uint32_t *>(base + w.offsets), base + w.valid,
                           reinterpret_cast<uint64_t *>(base + w.payload),
                           reinterpret_cast<uint64_t *>(base + w.chunk_off),
                           reinterpret_cast<uint32_t *>(base + w.fits),
                           reinterpret_cast<uint32_t *>(base + w.spare), base + w.scratch, out,
                           out_cap, chunk_offsets_out, dev_status, stream);
  return hip_status(e);
}

uint64_t kvc_decode_refined_ws_bytes(const kvc_codec_desc *dd, uint32_t n_chunks) {
  if (!desc_ok(dd)) return 0;
  return 2 * ws_layout(to_desc(dd), n_chunks, false).total;
}

kvc_status kvc_decode_refined(const kvc_codec_desc *dd, const void *tables, const void *rtables,
                              uint32_t refine_bits, const kvc_refined_chunk_ref *chunks,
                              uint32_t n_chunks, uint16_t *kv_out, uint32_t T_total, void *ws,
                              uint64_t ws_bytes, int32_t *dev_status, hipStream_t stream) {
  if (!desc_ok(dd) || !refine_bits_ok(refine_bits)) return KVC_ERR_INVALID_ARG;
  const Desc d = to_desc(dd);
  if (!tables || !aligned(tables, 16) || !rtables || !aligned(rtables, 16) || !dev_status ||
      !aligned(dev_status, 4))
    return KVC_ERR_INVALID_ARG;
  if (n_chunks > 65535) return KVC_ERR_SHAPE;
  if (n_chunks && (!chunks || !kv_out || !aligned(kv_out, 2))) return KVC_ERR_INVALID_ARG;
  const WsLayout w = ws_layout(d, n_chunks, false);
  if (n_chunks && (!ws || !aligned(ws, 256))) return KVC_ERR_INVALID_ARG;
  if (ws_bytes < 2 * w.total) return KVC_ERR_CAPACITY;
  const uint64_t S = n_streams(d);
  std::vector<std::pair<ChunkInfo, ChunkInfo>> info(n_chunks);
  std::vector<std::pair<uint32_t, uint32_t>> ranges(n_chunks);
  for (uint32_t k = 0; k < n_chunks; ++k) {
    const kvc_refined_chunk_ref &c = chunks[k];
    if (!c.container || !aligned(c.container, 4) || !c.refinement || !aligned(c.refinement, 4))
      return KVC_ERR_INVALID_ARG;
    if (c.level >= d.nlev || c.reserved != 0) return KVC_ERR_INVALID_ARG;
    if (c.n_tokens < 1 || c.n_tokens > d.chunk) return KVC_ERR_SHAPE;
    if ((uint64_t)c.first_token + c.n_tokens > T_total) return KVC_ERR_SHAPE;
    for (const uint64_t nb : {c.container_bytes, c.refinement_bytes})
      if (nb < kHdrBytes + kRecBytes * S || nb > 0xFFFFFFFFull) return KVC_ERR_SHAPE;
    ChunkInfo b{}, r{};
    b.cont = c.container;
    b.records = c.container + kHdrBytes;
    b.cont_bytes = c.container_bytes;
    r.cont = c.refinement;
    r.records = c.refinement + kHdrBytes;
    r.cont_bytes = c.refinement_bytes;
    b.first_token = r.first_token = c.first_token;
    b.n_tokens = r.n_tokens = c.n_tokens;
    b.level = r.level = c.level;
    b.out_tokens = r.out_tokens = T_total;
    b.out = r.out = kv_out;
    info[k] = {b, r};
    ranges[k] = {c.first_token, c.first_token + c.n_tokens};
  }
  std::sort(ranges.begin(), ranges.end());
  for (uint32_t k = 1; k < n_chunks; ++k)
    if (ranges[k].first < ranges[k - 1].second) return KVC_ERR_SHAPE;
  // decode groups as in kvc_decode: the chunk table ordered by level, split
  // into near-equal groups (one workgroup per (row, channel block) and group,
  // each wave taking at most kMaxRounds chunks); a workgroup stages, for
  // every level its group holds, the base delta models and both refinement
  // models
  std::stable_sort(info.begin(), info.end(),
                   [](const std::pair<ChunkInfo, ChunkInfo> &a,
                      const std::pair<ChunkInfo, ChunkInfo> &b) { return a.first.level < b.first.level; });
  constexpr uint32_t kMaxRounds = 4;
  constexpr size_t kRefinedLdsBudget = 160u * 1024u;
  uint32_t all_levels = 0;
  for (const auto &c : info) all_levels |= 1u << c.first.level;
  const uint32_t lv_all = (uint32_t)__builtin_popcount(all_levels);
  uint32_t wmax = 1;
  for (uint32_t wv = kDecodeMaxWaves; wv >= 1; --wv)
    if (decode_refined_lds_bytes(lv_all, refine_bits, wv) <= kRefinedLdsBudget) {
      wmax = wv;
      break;
    }
  std::vector<DecodeGroup> groups;
  uint32_t levels = 1, waves = 1;
  const uint32_t ng = (n_chunks + wmax * kMaxRounds - 1) / (wmax * kMaxRounds);
  for (uint32_t gi = 0; gi < ng; ++gi) {
    const uint32_t a = (uint32_t)((uint64_t)n_chunks * gi / ng);
    const uint32_t b = (uint32_t)((uint64_t)n_chunks * (gi + 1) / ng);
    DecodeGroup g{};
    g.start = a;
    g.count = b - a;
    for (uint32_t i = a; i < b; ++i) g.level |= 1u << info[i].first.level;
    levels = std::max<uint32_t>(levels, (uint32_t)__builtin_popcount(g.level));
    waves = std::max<uint32_t>(waves, std::min<uint32_t>(wmax, g.count));
    groups.push_back(g);
  }
  hipError_t e = launch_reset_status(dev_status, stream);
  if (e != hipSuccess || n_chunks == 0) return hip_status(e);
  std::vector<ChunkInfo> bi(n_chunks), ri(n_chunks);
  for (uint32_t k = 0; k < n_chunks; ++k) {
    bi[k] = info[k].first;
    ri[k] = info[k].second;
  }
  uint8_t *wb = static_cast<uint8_t *>(ws), *wr = wb + w.total;
  ChunkInfo *dbch = reinterpret_cast<ChunkInfo *>(wb + w.chunks);
  ChunkInfo *drch = reinterpret_cast<ChunkInfo *>(wr + w.chunks);
  e = launch_load_chunks(bi.data(), n_chunks, dbch, reinterpret_cast<uint32_t *>(wb + w.hdr), stream);
  if (e == hipSuccess)
    e = launch_load_chunks(ri.data(), n_chunks, drch, reinterpret_cast<uint32_t *>(wr + w.hdr), stream);
  if (e == hipSuccess)
    e = launch_index(d, dbch, n_chunks, reinterpret_cast<uint64_t *>(wb + w.rows),
                     reinterpret_cast<uint32_t *>(wb + w.hdr),
                     reinterpret_cast<uint32_t *>(wb + w.offsets), wb + w.valid,
                     reinterpret_cast<uint64_t *>(wb + w.payload),
                     static_cast<const uint8_t *>(tables), 1, dev_status, stream);
  if (e == hipSuccess)
    e = launch_index(d, drch, n_chunks, reinterpret_cast<uint64_t *>(wr + w.rows),
                     reinterpret_cast<uint32_t *>(wr + w.hdr),
                     reinterpret_cast<uint32_t *>(wr + w.offsets), wr + w.valid,
                     reinterpret_cast<uint64_t *>(wr + w.payload),
                     static_cast<const uint8_t *>(rtables), 2, dev_status, stream);
  if (e != hipSuccess) return KVC_ERR_HIP;
  DecodeGroup *dgr = reinterpret_cast<DecodeGroup *>(wb + w.groups);
  e = launch_load_groups(groups.data(), (uint32_t)groups.size(), dgr, stream);
  if (e != hipSuccess) return KVC_ERR_HIP;
  e = launch_decode_refined(d, refine_bits, dbch, drch, dgr, (uint32_t)groups.size(), levels,
                            waves,
                            wb + w.valid, wr + w.valid,
                            reinterpret_cast<uint32_t *>(wb + w.offsets),
                            reinterpret_cast<uint32_t *>(wr + w.offsets),
                            static_cast<const uint8_t *>(tables),
                            static_cast<const uint8_t *>(rtables), dev_status, stream);
  return hip_status(e);
}

uint64_t kvc_restore_staging_bytes(const kvc_host_chunk *chunks, uint32_t n_chunks,
                                   uint32_t batch_chunks) {
  if (!chunks || n_chunks == 0 || batch_chunks == 0) return 0;
  const uint32_t nb = (n_chunks + batch_chunks - 1) / batch_chunks;
  return restore_slot_bytes(chunks, n_chunks, batch_chunks) * std::min(nb, kRestoreSlots);
}

kvc_status kvc_restore(const kvc_codec_desc *dd, const void *tables, const kvc_host_chunk *chunks,
                       uint32_t n_chunks, uint32_t batch_chunks, uint16_t *kv_out,
                       uint32_t T_total, uint8_t *staging, uint64_t staging_bytes, void *ws,
                       uint64_t ws_bytes, int32_t *dev_status, hipStream_t compute,
                       hipStream_t copy, hipEvent_t *batch_done) {
  // every check of every batch before anything is queued
  if (!desc_ok(dd)) return KVC_ERR_INVALID_ARG;
  const Desc d = to_desc(dd);
  if (!tables || !aligned(tables, 16) || !dev_status || !aligned(dev_status, 4))
    return KVC_ERR_INVALID_ARG;
  if (batch_chunks == 0) return KVC_ERR_INVALID_ARG;
  if (n_chunks > 65535) return KVC_ERR_SHAPE;
  if (n_chunks == 0) return hip_status(launch_reset_status(dev_status, compute));
  if (!chunks || !kv_out || !aligned(kv_out, 2) || !staging || !aligned(staging, 256))
    return KVC_ERR_INVALID_ARG;
  if (!ws || !aligned(ws, 256)) return KVC_ERR_INVALID_ARG;
  const uint64_t S = n_streams(d);
  std::vector<std::pair<uint32_t, uint32_t>> ranges(n_chunks);
  for (uint32_t k = 0; k < n_chunks; ++k) {
    const kvc_host_chunk &c = chunks[k];
    if (!c.host_container || c.level >= d.nlev || c.reserved != 0) return KVC_ERR_INVALID_ARG;
    if (c.n_tokens < 1 || c.n_tokens > d.chunk) return KVC_ERR_SHAPE;
    if ((uint64_t)c.first_token + c.n_tokens > T_total) return KVC_ERR_SHAPE;
    if (c.container_bytes < kHdrBytes + kRecBytes * S) return KVC_ERR_SHAPE;
    if (c.container_bytes > 0xFFFFFFFFull) return KVC_ERR_SHAPE;
    ranges[k] = {c.first_token, c.first_token + c.n_tokens};
  }
  std::sort(ranges.begin(), ranges.end());
  for (uint32_t k = 1; k < n_chunks; ++k)
    if (ranges[k].first < ranges[k - 1].second) return KVC_ERR_SHAPE;
  const uint32_t per = std::min(batch_chunks, n_chunks);
  const uint32_t nb = (n_chunks + per - 1) / per;
  const uint64_t slot = restore_slot_bytes(chunks, n_chunks, per);
  if (staging_bytes < slot * std::min(nb, kRestoreSlots)) return KVC_ERR_CAPACITY;
  if (ws_bytes < ws_layout(d, per, false).total) return KVC_ERR_CAPACITY;

  RestoreEvents evs;  // per slot: copied, decoded; then the start
  if (evs.create() != hipSuccess) return KVC_ERR_HIP;
  hipEvent_t *copied = evs.ev, *decoded = evs.ev + kRestoreSlots;
  hipEvent_t start = evs.ev[2 * kRestoreSlots];
  hipError_t e = launch_reset_status(dev_status, compute);
  // the staging slots may still be read by work queued earlier on compute
  if (e == hipSuccess) e = hipEventRecord(start, compute);
  if (e == hipSuccess) e = hipStreamWaitEvent(copy, start, 0);
  if (e != hipSuccess) return KVC_ERR_HIP;
  std::vector<kvc_chunk_ref> refs;
  for (uint32_t b = 0; b < nb; ++b) {
    const uint32_t s = b % kRestoreSlots, k0 = b * per, k1 = std::min(n_chunks, k0 + per);
    uint8_t *base = staging + (uint64_t)s * slot;
    if (b >= kRestoreSlots && hipStreamWaitEvent(copy, decoded[s], 0) != hipSuccess)
      return KVC_ERR_HIP;
    refs.clear();
    uint64_t off = 0;
    for (uint32_t k = k0; k < k1; ++k) {
      const kvc_host_chunk &c = chunks[k];
      if (hipMemcpyAsync(base + off, c.host_container, c.container_bytes, hipMemcpyHostToDevice,
                         copy) != hipSuccess)
        return KVC_ERR_HIP;
      refs.push_back({base + off, c.container_bytes, c.first_token, c.n_tokens, c.level, 0});
      off += align256(c.container_bytes);
    }
    if (hipEventRecord(copied[s], copy) != hipSuccess ||
        hipStreamWaitEvent(compute, copied[s], 0) != hipSuccess)
      return KVC_ERR_HIP;
    const kvc_status st = decode_common(dd, tables, refs.data(), (uint32_t)refs.size(), kv_out,
                                        T_total, ws, ws_bytes, dev_status, compute, 0, nullptr,
                                        /*reset_status=*/false);
    if (st != KVC_OK) return st;
    if (hipEventRecord(decoded[s], compute) != hipSuccess) return KVC_ERR_HIP;
    if (batch_done && hipEventRecord(batch_done[b], compute) != hipSuccess) return KVC_ERR_HIP;
  }
  return KVC_OK;
}

}  // extern "C"
