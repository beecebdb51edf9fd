// Plan of the ring-buffer minibatch pipeline: how the expert-sorted rows are
// cut into minibatches, which tasks each minibatch brings, in which order the
// persistent kernel hands them out, and what each task waits for.
//
// The pages process the dispatched tokens in tunable minibatches taken from a
// fixed ring token buffer (the macrobatch), with the GPU itself driving the
// state and no host synchronisation in between (kucoin.com, "Cursor's MoK
// réalise une amélioration des performances de 2,37x sur NVIDIA GB300
// NVL72", section 02; fluidifia.com, "Cursor ouvre MoK, un mégakernel qui
// accélère l'entraînement MoE", section "Comment MoK tente de gratter des
// millisecondes partout").
//
// Everything here is plain integer arithmetic on host or device
// (__host__ __device__), so that the CPU model of the scheduler runs exactly
// the code the GPU runs.
#pragma once
#include <stdint.h>

#if defined(__HIPCC__)
#define MOK_HD __host__ __device__ __forceinline__
#else
#define MOK_HD inline
#endif

namespace mok {
namespace ring {

constexpr int kTileRows = 256;     // row-tile height of the ring's GEMM tiles
constexpr int kCopyRows = 32;      // rows per copy task (the mover's unit)
constexpr int kCombTokens = 16;    // tokens per combine task
// Task kinds; a phase lists its tasks in this order.
enum Kind { COPY = 0, UP = 1, DOWN = 2, COMB = 3, NKIND = 4 };
// Phase lag of each kind: phase p holds COPY(p), UP(p - 1), DOWN(p - 3) and
// the combine list of minibatch p - 4, so that a task's inputs were handed
// out at least one phase (about one machine-wide round of tasks) earlier.
constexpr int kLag[NKIND] = {0, 1, 3, 4};

// Largest number of minibatches the partition below can make from P rows.
MOK_HD int64_t max_minibatches(int64_t P, int R) { return 2 * ((P + R - 1) / R) + 2; }

// Cut the local experts' rows into minibatches of at most R rows (R a
// multiple of kTileRows), in expert order: whole experts while they fit, an
// expert with more than R rows in pieces of R rows (the last piece may take
// the following experts along).  Every boundary is then a row-tile boundary
// of the whole-layer tiling (tiles of kTileRows rows from each expert's
// first row), so no tile is split.
//   off   [E_loc + 1] local expert offsets (off[0] = 0, off[E_loc] = P)
//   tp    [E_loc + 1] prefix of each expert's kTileRows-row tiles
//   mb_row, mb_tile [M + 1]: first row and first row tile of minibatch m
// Returns M (0 when there are no rows).
MOK_HD int partition(const int32_t* off, const int32_t* tp, int E_loc, int R, int32_t* mb_row, int32_t* mb_tile) {
  int M = 0, cur = 0;
  mb_row[0] = off[0];
  mb_tile[0] = tp[0];
  for (int i = 0; i < E_loc; ++i) {
    const int n = off[i + 1] - off[i];
    if (n <= 0) continue;
    if (n <= R) {
      if (cur > 0 && cur + n > R) {
        ++M;
        mb_row[M] = off[i];
        mb_tile[M] = tp[i];
        cur = 0;
      }
      cur += n;
    } else {
      if (cur > 0) {
        ++M;
        mb_row[M] = off[i];
        mb_tile[M] = tp[i];
        cur = 0;
      }
      int c = 0;
      while (n - c > R) {
        c += R;
        ++M;
        mb_row[M] = off[i] + c;
        mb_tile[M] = tp[i] + c / kTileRows;
      }
      cur = n - c;
    }
  }
  if (cur > 0) {
    ++M;
    mb_row[M] = off[E_loc];
    mb_tile[M] = tp[E_loc];
  }
  return M;
}

// Minibatch holding row r (mb_row[m] <= r < mb_row[m + 1]), 0 <= r < P.
MOK_HD int minibatch_of_row(const int32_t* mb_row, int M, int r) {
  int lo = 0, hi = M - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (mb_row[mid] <= r) lo = mid; else hi = mid - 1;
  }
  return lo;
}

// Phases of the task sequence: a combine list c (0: tokens without a local
// pair; m + 1: tokens whose last local pair lies in minibatch m) sits in
// phase c + kLag[COMB] - 1, so NP = M + kLag[COMB] phases hold everything.
MOK_HD int num_phases(int M) { return M + kLag[COMB]; }

// Task count of slot (phase p, kind) given the minibatch sizes.
struct Sizes {
  const int32_t* mb_row;   // [M + 1]
  const int32_t* mb_tile;  // [M + 1]
  const int32_t* comb_n;   // [M + 1] tokens per combine list
  int M, ntn_up, ntn_dn;
};
MOK_HD int slot_tasks(const Sizes& z, int p, int kind) {
  if (kind == COMB) {
    const int c = p - kLag[COMB] + 1;  // combine list index
    if (c < 0 || c > z.M) return 0;
    return (z.comb_n[c] + kCombTokens - 1) / kCombTokens;
  }
  const int m = p - kLag[kind];
  if (m < 0 || m >= z.M) return 0;
  if (kind == COPY) return (z.mb_row[m + 1] - z.mb_row[m] + kCopyRows - 1) / kCopyRows;
  const int tiles = z.mb_tile[m + 1] - z.mb_tile[m];
  return tiles * (kind == UP ? z.ntn_up : z.ntn_dn);
}

// A decoded task: its kind, minibatch (combine: list index - 1) and index
// within the slot.
struct Task {
  int kind, m, local;
};
// pref [NKIND * NP + 1]: prefix of slot_tasks over slots q = NKIND * p + kind.
MOK_HD Task decode(const int32_t* pref, int nslots, int t) {
  int lo = 0, hi = nslots - 1;  // last slot q with pref[q] <= t
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (pref[mid] <= t) lo = mid; else hi = mid - 1;
  }
  Task k;
  k.kind = lo % NKIND;
  const int p = lo / NKIND;
  k.m = k.kind == COMB ? p - kLag[COMB] : p - kLag[k.kind];
  k.local = t - pref[lo];
  return k;
}
// Tasks of (kind, minibatch m) from the prefix (combine: list m + 1).
MOK_HD int count_of(const int32_t* pref, int kind, int m) {
  const int q = NKIND * (m + kLag[kind]) + kind;
  return pref[q + 1] - pref[q];
}

// What a task waits for, as one or more (counter kind, minibatch) pairs that
// must reach count_of(): COPY(m) waits until UP(m - S) has read the ring slot
// it reuses; UP(m) waits for COPY(m); DOWN(m) for UP(m) (all columns of H);
// the combine list of minibatch m waits for DOWN(m') for every m' <= m (a
// token's pairs lie in minibatches up to its last one).  Returns the number of
// single-counter waits; for the combine the caller walks m' = its frontier .. m.
MOK_HD int wait_of(const Task& k, int S, int* wkind, int* wm) {
  switch (k.kind) {
    case COPY:
      if (k.m >= S) { *wkind = UP; *wm = k.m - S; return 1; }
      return 0;
    case UP: *wkind = COPY; *wm = k.m; return 1;
    case DOWN: *wkind = UP; *wm = k.m; return 1;
    default: return 0;  // combine: see above
  }
}

}  // namespace ring
}  // namespace mok
