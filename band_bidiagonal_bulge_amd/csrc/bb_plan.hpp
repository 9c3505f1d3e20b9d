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

// Working band: element (i, j) at band[i*stride + (j - i + sub)], with room
// for the bulge: sub = t of the first pass diagonals below the main diagonal
// and bw + sub above it (nonzeros of a pass with (b, t) never leave that
// range), ld = bw + 2 sub + 1 entries in use per row.  The row stride pads ld
// to a multiple of 16 bytes: rows are whole 16-byte units (vector copies of
// row ranges), and stride - 1 is odd, so lanes reading one row each at the
// same column hit distinct LDS banks.
struct Geometry {
  int64_t n = 0;
  int32_t bw = 0, tw = 0, dtype = 0, esize = 0;
  int32_t sub = 0, ld = 0, maxt = 0;
  int32_t stride = 0;      // elements between rows of the working band
  size_t band_bytes = 0;   // n * stride * esize, rounded up to 256
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
  g.esize = dtype == 1 ? 8 : (dtype == 2 ? 2 : 4);
  g.maxt = bw > 1 ? std::min(tw, bw - 1) : 0;
  g.sub = g.maxt;
  g.ld = g.sub + bw + g.maxt + 1;
  const int32_t per16 = 16 / g.esize;
  g.stride = (g.ld + per16 - 1) / per16 * per16;
  g.band_bytes = (size_t(n) * size_t(g.stride) * size_t(g.esize) + 255) / 256 * 256;
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

// Half-cycle lag between consecutive sweeps: 2 when b' >= 3, 3 when b' = 2,
// 4 when b' = 1.
inline int lag_of(const Pass &p) {
  const int bp = p.b - p.t;
  return bp >= 3 ? 2 : (bp == 2 ? 3 : 4);
}

// Rows a sweep touches in half-cycle q (2k: row half, 2k+1: column half):
// [lo, hi].
inline void half_rows(int64_t n, const Pass &p, int64_t R, int64_t q, int64_t *lo, int64_t *hi) {
  const int64_t k = q >> 1;
  const int64_t c = R + (p.b - p.t) + k * p.b;
  *hi = std::min<int64_t>(c + p.t, n - 1);
  *lo = (q & 1) ? c : (k == 0 ? R : c - p.b);
}

// Ring rows a sweep group of G needs so that it always makes progress.  In a
// state where no wave can move, each wave waits for its predecessor with
// exactly d-1 half-cycles of lag in completed halves (or for rows); the ring
// must then hold every row from the lowest row any wave will still touch to
// the highest row any wave needs.  Bounded from above by taking the rows
// needed at lag d-1 and the lowest rows at lag d, over every group and step.
inline int64_t group_ring_rows(int64_t n, const Pass &p, int G) {
  const int64_t ns = sweeps_of(n, p);
  const int d = lag_of(p);
  int64_t need = 0;
  std::vector<int64_t> K(size_t(G), 0);
  for (int64_t R0 = 0; R0 < ns; R0 += G) {
    const int Gg = int(std::min<int64_t>(G, ns - R0));
    int64_t steps = 0;
    for (int j = 0; j < Gg; ++j) {
      K[size_t(j)] = cycles_of(n, p, R0 + j);
      steps = std::max<int64_t>(steps, 2 * K[size_t(j)] + int64_t(j) * d);
    }
    for (int64_t q0 = 0; q0 < steps; ++q0) {
      int64_t hi = -1, fl = n;
      for (int j = 0; j < Gg; ++j) {
        const int64_t R = R0 + j, twoK = 2 * K[size_t(j)];
        int64_t lo, h;
        const int64_t qa = q0 - int64_t(j) * (d - 1);  // most advanced position: rows needed
        if (qa >= 0 && qa < twoK) {
          half_rows(n, p, R, qa, &lo, &h);
          hi = std::max(hi, h);
        }
        const int64_t qb = q0 - int64_t(j) * d;  // least advanced position: rows still live
        if (qb < 0) {
          fl = std::min(fl, R);
        } else if (qb < twoK) {
          half_rows(n, p, R, qb, &lo, &h);
          fl = std::min(fl, lo);
        }
      }
      if (hi >= 0) need = std::max(need, hi - fl + 1);
    }
  }
  return need;
}

// Symmetric band -> tridiagonal: the upper triangle of the band with room
// for the fill, which reaches bw + T superdiagonals (T = t of the first
// pass).  Element (i, j), 0 <= j-i <= W = bw + T, at band[i*stride + j-i];
// stride = W+1 padded to 16 bytes.  Counters follow as for the general band.
struct SymGeometry {
  int64_t n = 0;
  int32_t bw = 0, tw = 0, dtype = 0, esize = 0;
  int32_t maxt = 0, W = 0, ld = 0, stride = 0;
  size_t band_bytes = 0, sync_offset = 0, sync_words = 0, total_bytes = 0;
};

inline SymGeometry make_sym_geometry(int64_t n, int32_t bw, int32_t tw, int32_t dtype) {
  SymGeometry g;
  g.n = n;
  g.bw = bw;
  g.tw = tw;
  g.dtype = dtype;
  g.esize = dtype == 1 ? 8 : (dtype == 2 ? 2 : 4);
  g.maxt = bw > 1 ? std::min(tw, bw - 1) : 0;
  g.W = bw + g.maxt;
  g.ld = g.W + 1;
  const int32_t per16 = 16 / g.esize;
  g.stride = (g.ld + per16 - 1) / per16 * per16;
  g.band_bytes = (size_t(n) * size_t(g.stride) * size_t(g.esize) + 255) / 256 * 256;
  g.sync_offset = g.band_bytes;
  g.sync_words = size_t(kSyncHeader + (n + 1) * kLine);
  g.total_bytes = g.sync_offset + (g.sync_words * 4 + 255) / 256 * 256;
  return g;
}

// The symmetric reduction runs by half-cycles too: half 2k forms cycle k's
// reflector and applies it to the pivot row and the row segments above the
// block (rows p..c-1), half 2k+1 applies it to the block and the column
// segments (rows c..ch).  The lag between consecutive sweeps is then
// lag_of(p) half-cycles, as for the general band (derived from the halves'
// read/write footprints), capped at all of the predecessor; a sweep
// publishes its final count after its predecessor's.

// Rows symmetric half-cycle q of sweep R touches: [lo, hi].
inline void sym_half_rows(int64_t n, const Pass &p, int64_t R, int64_t q, int64_t *lo, int64_t *hi) {
  const int64_t k = q >> 1;
  const int64_t c = R + (p.b - p.t) + k * p.b;
  if (q & 1) {
    *lo = c;
    *hi = std::min<int64_t>(c + p.t, n - 1);
  } else {
    *lo = k == 0 ? R : c - p.b;
    *hi = c - 1;
  }
}

// Ring rows a group of G symmetric sweeps needs (the bound of
// group_ring_rows with the symmetric halves).
inline int64_t sym_group_ring_rows(int64_t n, const Pass &p, int G) {
  const int64_t ns = sweeps_of(n, p);
  const int d = lag_of(p);
  int64_t need = 0;
  std::vector<int64_t> K(size_t(G), 0);
  for (int64_t R0 = 0; R0 < ns; R0 += G) {
    const int Gg = int(std::min<int64_t>(G, ns - R0));
    int64_t steps = 0;
    for (int j = 0; j < Gg; ++j) {
      K[size_t(j)] = cycles_of(n, p, R0 + j);
      steps = std::max<int64_t>(steps, 2 * K[size_t(j)] + int64_t(j) * d);
    }
    for (int64_t q0 = 0; q0 < steps; ++q0) {
      int64_t hi = -1, fl = n;
      for (int j = 0; j < Gg; ++j) {
        const int64_t R = R0 + j, twoK = 2 * K[size_t(j)];
        int64_t lo, h;
        const int64_t qa = q0 - int64_t(j) * (d - 1);  // most advanced position: rows needed
        if (qa >= 0 && qa < twoK) {
          sym_half_rows(n, p, R, qa, &lo, &h);
          hi = std::max(hi, h);
        }
        const int64_t qb = q0 - int64_t(j) * d;  // least advanced position: rows still live
        if (qb < 0) {
          fl = std::min(fl, R);
        } else if (qb < twoK) {
          sym_half_rows(n, p, R, qb, &lo, &h);
          fl = std::min(fl, lo);
        }
      }
      if (hi >= 0) need = std::max(need, hi - fl + 1);
    }
  }
  return need;
}

}  // namespace bb
