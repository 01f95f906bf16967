// Per-chunk compression-level choice for streaming a context over a link of
// varying bandwidth (host code only).
//
// CacheGen page, 核心方法 (online streaming paragraph): before each chunk
// the sender estimates the time the remaining chunks need from the last
// chunk's measured throughput and sends the chunk at the best-quality level
// for which that estimate still meets the TTFT SLO; 关键观察, assumption 1:
// the estimate trails the link by at most one chunk.  The link is a
// piecewise-constant bandwidth trace; the result is each chunk's level and
// arrival time.
#include <cmath>
#include <cstdint>

#include "kvc.h"

namespace {

// Time at which `bytes` sent from time t over the trace have arrived.
double transfer_end(const kvc_bw_piece *trace, uint32_t n_pieces, double t, double bytes) {
  uint32_t k = 0;
  while (k + 1 < n_pieces && trace[k + 1].start_s <= t) ++k;
  for (;; ++k) {
    const double rate = trace[k].bytes_per_s;
    if (k + 1 == n_pieces) return t + bytes / rate;
    const double avail = (trace[k + 1].start_s - t) * rate;
    if (bytes <= avail) return t + bytes / rate;
    bytes -= avail;
    t = trace[k + 1].start_s;
  }
}

bool positive_finite(double x) { return std::isfinite(x) && x > 0.0; }

}  // namespace

extern "C" kvc_status kvc_plan_stream(const uint64_t *chunk_bytes, uint32_t n_chunks,
                                      uint32_t n_levels, const kvc_bw_piece *trace,
                                      uint32_t n_pieces, double slo_s, double init_bytes_per_s,
                                      uint8_t *levels_out, double *finish_s_out) {
  if (n_chunks == 0) return KVC_OK;
  if (!chunk_bytes || !trace || !levels_out || !finish_s_out) return KVC_ERR_INVALID_ARG;
  if (n_levels < 1 || n_levels > 255 || n_pieces < 1) return KVC_ERR_INVALID_ARG;
  if (!std::isfinite(slo_s) || !positive_finite(init_bytes_per_s)) return KVC_ERR_INVALID_ARG;
  if (trace[0].start_s != 0.0) return KVC_ERR_INVALID_ARG;
  for (uint32_t k = 0; k < n_pieces; ++k) {
    if (!positive_finite(trace[k].bytes_per_s)) return KVC_ERR_INVALID_ARG;
    if (k && !(trace[k].start_s > trace[k - 1].start_s && std::isfinite(trace[k].start_s)))
      return KVC_ERR_INVALID_ARG;
  }
  double t = 0.0, estimate = init_bytes_per_s;
  for (uint32_t i = 0; i < n_chunks; ++i) {
    // bytes still to send at each level, this chunk included (exact sums)
    uint32_t choice = n_levels;
    uint32_t smallest = 0;
    uint64_t smallest_bytes = UINT64_MAX;
    for (uint32_t l = 0; l < n_levels; ++l) {
      uint64_t rest = 0;
      for (uint32_t j = i; j < n_chunks; ++j) rest += chunk_bytes[(uint64_t)j * n_levels + l];
      if (rest < smallest_bytes) {
        smallest_bytes = rest;
        smallest = l;
      }
      if (choice == n_levels && t + (double)rest / estimate <= slo_s) choice = l;
    }
    if (choice == n_levels) choice = smallest;
    const double bytes = (double)chunk_bytes[(uint64_t)i * n_levels + choice];
    const double end = transfer_end(trace, n_pieces, t, bytes);
    levels_out[i] = (uint8_t)choice;
    finish_s_out[i] = end;
    // the next estimate: this chunk's throughput (a chunk of 0 bytes, or one
    // too small to take any time, leaves the estimate as it was)
    if (end > t && bytes > 0.0) estimate = bytes / (end - t);
    t = end;
  }
  return KVC_OK;
}
