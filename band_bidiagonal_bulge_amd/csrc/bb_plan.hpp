// Host-side planning of a band -> bidiagonal reduction: pass list, sweep and
// cycle counts, the working-band geometry and the workspace layout.
//
// Successive band reduction (page "Accelerating Bidiagonalization of Banded
// Matrices through Memory-Aware Bulge-Chasing on GPUs", tile-width
// definition): a pass takes bandwidth b to b - t, t = min(TW, b-1), so the
// last pass lands on 1.  In a pass, sweep R = 0 .. n-b'-2 runs cycles
// k = 0, 1, ... while c = R + b' + k b <= n-2.
#pragma once

#include <algorithm>
#include <cstddef>
#include <cstdint>
#include <vector>

namespace bb {

struct Pass {
  int32_t b;  // bandwidth entering the pass
  int32_t t;  // diagonals removed (tile width, clamped to b-1)
};

inline std::vector<Pass> pass_list(int32_t bw, int32_t tw) {
  std::vector<Pass> out;
  for (int32_t b = bw; b > 1;) {
    const int32_t t = std::min(tw, b - 1);
    out.push_back({b, t});
    b -= t;
  }
  return out;
}

// Sweeps of a pass: rows R whose first cycle exists (c = R + b' <= n-2).
inline int64_t sweeps_of(int64_t n, const Pass &p) {
  const int64_t bp = p.b - p.t;
  return std::max<int64_t>(0, n - bp - 1);
}

// Cycles of sweep R: k = 0 .. K-1 with R + b' + k b <= n-2.
inline int64_t cycles_of(int64_t n, const Pass &p, int64_t R) {
  const int64_t last = n - 2 - R - (p.b - p.t);
  return last < 0 ? 0 : last / p.b + 1;
}

// Steps of a one-launch-per-step schedule with stagger s: max_R (s R + K_R).
inline int64_t steps_of(int64_t n, const Pass &p, int32_t s) {
  const int64_t ns = sweeps_of(n, p);
  int64_t best = 0;
  // s R + K_R is maximised near the last sweeps; K_R is non-increasing, so a
  // scan from the top until s R + max K cannot win suffices, but the plain
  // scan is cheap enough for the host.
  for (int64_t R = 0; R < ns; ++R) best = std::max(best, s * R + cycles_of(n, p, R));
  return best;
}

// Working band: element (i, j) at band[i*ld + (j - i + sub)], with room for
// the bulge: sub = t of the first pass diagonals below the main diagonal and
// bw + sub above it (nonzeros of a pass with (b, t) never leave that range).
struct Geometry {
  int64_t n = 0;
  int32_t bw = 0, tw = 0, dtype = 0, esize = 0;
  int32_t sub = 0, ld = 0, maxt = 0;
  size_t band_bytes = 0;   // n * ld * esize, rounded up to 256
  size_t sync_offset = 0;  // byte offset of the counters
  size_t sync_words = 0;   // 32-bit words of counters
  size_t total_bytes = 0;
};

// Counter area (32-bit words).  Every counter that one workgroup writes and
// others poll sits alone in a 128-byte cache line (kLine words), so a store
// to one never disturbs the line another workgroup is polling:
//   [0] device status; [kClaim] sweep claim counter; [kProf ..] profiling
//   counters (instrumented builds); [kSyncHeader + R*kLine] progress of sweep R.
constexpr int64_t kLine = 32;
constexpr int64_t kClaim = kLine;
constexpr int64_t kProf = 2 * kLine;
constexpr int64_t kSyncHeader = 4 * kLine;

inline Geometry make_geometry(int64_t n, int32_t bw, int32_t tw, int32_t dtype) {
  Geometry g;
  g.n = n;
  g.bw = bw;
  g.tw = tw;
  g.dtype = dtype;
  g.esize = dtype == 1 ? 8 : 4;
  g.maxt = bw > 1 ? std::min(tw, bw - 1) : 0;
  g.sub = g.maxt;
  g.ld = g.sub + bw + g.maxt + 1;
  g.band_bytes = (size_t(n) * size_t(g.ld) * size_t(g.esize) + 255) / 256 * 256;
  g.sync_offset = g.band_bytes;
  g.sync_words = size_t(kSyncHeader + (n + 1) * kLine);
  g.total_bytes = g.sync_offset + (g.sync_words * 4 + 255) / 256 * 256;
  return g;
}

// Work of one cycle: m = ch-c+1 columns of the row block (rows r..ch) and
// rows of the column block (columns c..jend).  Algorithmic elements U =
// m * (rows + cols - m): the union of the two blocks, each read and written
// once.
struct CycleShape {
  int64_t m, rows, cols;
};

inline CycleShape cycle_shape(int64_t n, const Pass &p, int64_t R, int64_t k) {
  const int64_t bp = p.b - p.t;
  const int64_t c = R + bp + k * p.b;
  const int64_t ch = std::min<int64_t>(c + p.t, n - 1);
  const int64_t r = k == 0 ? R : c - p.b;
  const int64_t jend = std::min<int64_t>(c + p.t + p.b, n - 1);
  return {ch - c + 1, ch - r + 1, jend - c + 1};
}

}  // namespace bb
