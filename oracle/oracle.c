/*
 * oracle.c -- plain, slow, CPU reference ("oracle") for one 3D Gaussian Splatting
 * training step: preprocess -> bin -> stable sort -> tile ranges -> forward blend ->
 * L1 loss -> backward blend -> preprocess backward -> Adam.
 *
 * TEST INFRASTRUCTURE ONLY.  This library is loaded by the test-suite, the smoke check
 * and the bench's CPU-baseline leg, nothing else.  It shares no code, header, table or
 * constant generator with the GPU library; the two meet only through the seeded inputs.
 *
 * What it follows.  The pages name the stages but print no formulas:
 *   [Scaling]  "Scaling 3D Gaussian Splatting with Distributed Compute: Why One GPU Is
 *              Never Enough" -- the parameter list (mean, covariance from scale and
 *              rotation, SH colour, opacity), the per-Gaussian projection to 2D means,
 *              depths, conics, radii and a visibility mask, SH evaluated to RGB before the
 *              exchange, the 12-scalar projected record, per-tile sorted intersection lists,
 *              per-tile offsets into the sorted list, rasterization by alpha compositing, the
 *              L1 term of the loss, gradients flowing back to mean, covariance, colour and
 *              opacity, and a local Adam step.
 *   [Iso]      "Toward Distributed 3D Gaussian Splatting for High-Resolution Isosurface
 *              Visualization", sections I and III (3D-GS of Kerbl et al. trained from
 *              synthetic orbit views).
 * Both cite 3D-GS (Kerbl et al. 2023); each formula below is the standard 3D-GS / EWA
 * splatting reading of the stage named, and every constant the pages leave open is listed
 * in the design notes with the reading taken.
 *
 * Arithmetic.  IEEE double throughout (compiled without -ffast-math, no FMA contraction).
 * Where a floating-point value decides an integer or a branch (tile radii, tile rects,
 * the alpha threshold, the transmittance cut-off, the opacity clamp), the value is rounded
 * to float32 and compared with the float32 constant, i.e. the decision is taken in the
 * precision of the GPU kernel.  Gradients are accumulated in double.
 *
 * Parameter rows (planar [R][n] double):
 *   0-2 mean mu, 3-5 log-scale l, 6-9 quaternion q = (w,x,y,z), 10 opacity logit a,
 *   11 + 3k + ch : SH coefficient k (k < (d+1)^2) of colour channel ch.
 * Camera (17 doubles): viewmat row-major 3x4 [Rc | t] world->camera (x right, y down,
 *   z forward), fx, fy, cx, cy, near.
 * Projected record (planar [10][n] double): u, v, depth, opacity, A, B, C, r, g, b;
 *   radii int32 [2][n]; tiles uint32 [n].  A culled Gaussian has all of these 0.
 */
#include <math.h>
#include <omp.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define TILE 16
#define PRJ_U 0
#define PRJ_V 1
#define PRJ_DEPTH 2
#define PRJ_OPAC 3
#define PRJ_A 4
#define PRJ_B 5
#define PRJ_C 6
#define PRJ_R 7
#define PRJ_G 8
#define PRJ_BL 9
#define PRJ_FIELDS 10

/* Standard 3D-GS constants (the pages name the mechanism, not the numbers). */
#define ALPHA_MIN_F (1.0f / 255.0f)  /* entries with alpha below this are skipped      */
#define ALPHA_MAX 0.99               /* alpha clamp                                    */
#define ALPHA_MAX_F 0.99f
#define T_MIN_F 1e-4f                /* stop before blending when T would drop below   */
#define DILATION 0.3                 /* EWA screen-space low-pass, px^2 on the diagonal */
#define GUARD 1.3                    /* guard band for x/z, y/z inside the Jacobian     */

int or_rows_for_degree(int d) { return 11 + 3 * (d + 1) * (d + 1); }

/* The OpenMP threads of the embarrassingly parallel loops below (timing runs set them). */
void or_set_num_threads(int n) { omp_set_num_threads(n > 0 ? n : 1); }
int or_get_max_threads(void) { return omp_get_max_threads(); }

/* ------------------------------------------------------------------------------------ */
/* camera                                                                               */
/* ------------------------------------------------------------------------------------ */
typedef struct {
  double Rc[3][3], t[3];
  double fx, fy, cx, cy, near_plane;
  int W, H, TX, TY;
  double centre[3]; /* camera centre in world space: -Rc^T t */
} cam_t;

static void load_cam(const double* c, int W, int H, cam_t* k) {
  for (int i = 0; i < 3; i++) {
    for (int j = 0; j < 3; j++) k->Rc[i][j] = c[4 * i + j];
    k->t[i] = c[4 * i + 3];
  }
  k->fx = c[12]; k->fy = c[13]; k->cx = c[14]; k->cy = c[15]; k->near_plane = c[16];
  k->W = W; k->H = H;
  k->TX = (W + TILE - 1) / TILE; k->TY = (H + TILE - 1) / TILE;
  for (int j = 0; j < 3; j++) {
    k->centre[j] = 0.0;
    for (int i = 0; i < 3; i++) k->centre[j] -= k->Rc[i][j] * k->t[i];
  }
}

/* ------------------------------------------------------------------------------------ */
/* real spherical harmonics, Condon-Shortley phase, l = 0..3, m = -l..l                  */
/* ------------------------------------------------------------------------------------ */
/* Y[k] for a unit vector (x, y, z); the constants are evaluated from their closed forms. */
static void sh_basis(int deg, double x, double y, double z, double* Y) {
  const double pi = M_PI;
  Y[0] = 0.5 / sqrt(pi);
  if (deg < 1) return;
  const double c1 = sqrt(3.0 / (4.0 * pi));
  Y[1] = -c1 * y;
  Y[2] = c1 * z;
  Y[3] = -c1 * x;
  if (deg < 2) return;
  const double c2a = 0.5 * sqrt(15.0 / pi), c2b = 0.25 * sqrt(5.0 / pi), c2c = 0.25 * sqrt(15.0 / pi);
  Y[4] = c2a * x * y;
  Y[5] = -c2a * y * z;
  Y[6] = c2b * (2.0 * z * z - x * x - y * y);
  Y[7] = -c2a * x * z;
  Y[8] = c2c * (x * x - y * y);
  if (deg < 3) return;
  const double c3a = 0.25 * sqrt(35.0 / (2.0 * pi)), c3b = 0.5 * sqrt(105.0 / pi),
               c3c = 0.25 * sqrt(21.0 / (2.0 * pi)), c3d = 0.25 * sqrt(7.0 / pi),
               c3e = 0.25 * sqrt(105.0 / pi);
  Y[9] = -c3a * y * (3.0 * x * x - y * y);
  Y[10] = c3b * x * y * z;
  Y[11] = -c3c * y * (4.0 * z * z - x * x - y * y);
  Y[12] = c3d * z * (2.0 * z * z - 3.0 * x * x - 3.0 * y * y);
  Y[13] = -c3c * x * (4.0 * z * z - x * x - y * y);
  Y[14] = c3e * z * (x * x - y * y);
  Y[15] = -c3a * x * (x * x - 3.0 * y * y);
}

/* Partial derivatives dY[k][0..2] = (dY/dx, dY/dy, dY/dz) of the polynomials above. */
static void sh_basis_grad(int deg, double x, double y, double z, double dY[16][3]) {
  const double pi = M_PI;
  for (int k = 0; k < 16; k++) dY[k][0] = dY[k][1] = dY[k][2] = 0.0;
  if (deg < 1) return;
  const double c1 = sqrt(3.0 / (4.0 * pi));
  dY[1][1] = -c1;
  dY[2][2] = c1;
  dY[3][0] = -c1;
  if (deg < 2) return;
  const double c2a = 0.5 * sqrt(15.0 / pi), c2b = 0.25 * sqrt(5.0 / pi), c2c = 0.25 * sqrt(15.0 / pi);
  dY[4][0] = c2a * y;            dY[4][1] = c2a * x;
  dY[5][1] = -c2a * z;           dY[5][2] = -c2a * y;
  dY[6][0] = -2.0 * c2b * x;     dY[6][1] = -2.0 * c2b * y;     dY[6][2] = 4.0 * c2b * z;
  dY[7][0] = -c2a * z;           dY[7][2] = -c2a * x;
  dY[8][0] = 2.0 * c2c * x;      dY[8][1] = -2.0 * c2c * y;
  if (deg < 3) return;
  const double c3a = 0.25 * sqrt(35.0 / (2.0 * pi)), c3b = 0.5 * sqrt(105.0 / pi),
               c3c = 0.25 * sqrt(21.0 / (2.0 * pi)), c3d = 0.25 * sqrt(7.0 / pi),
               c3e = 0.25 * sqrt(105.0 / pi);
  /* Y9 = -c3a (3x^2 y - y^3) */
  dY[9][0] = -c3a * 6.0 * x * y;
  dY[9][1] = -c3a * (3.0 * x * x - 3.0 * y * y);
  /* Y10 = c3b xyz */
  dY[10][0] = c3b * y * z; dY[10][1] = c3b * x * z; dY[10][2] = c3b * x * y;
  /* Y11 = -c3c (4 y z^2 - x^2 y - y^3) */
  dY[11][0] = -c3c * (-2.0 * x * y);
  dY[11][1] = -c3c * (4.0 * z * z - x * x - 3.0 * y * y);
  dY[11][2] = -c3c * (8.0 * y * z);
  /* Y12 = c3d (2 z^3 - 3 x^2 z - 3 y^2 z) */
  dY[12][0] = c3d * (-6.0 * x * z);
  dY[12][1] = c3d * (-6.0 * y * z);
  dY[12][2] = c3d * (6.0 * z * z - 3.0 * x * x - 3.0 * y * y);
  /* Y13 = -c3c (4 x z^2 - x^3 - x y^2) */
  dY[13][0] = -c3c * (4.0 * z * z - 3.0 * x * x - y * y);
  dY[13][1] = -c3c * (-2.0 * x * y);
  dY[13][2] = -c3c * (8.0 * x * z);
  /* Y14 = c3e (x^2 z - y^2 z) */
  dY[14][0] = c3e * 2.0 * x * z;
  dY[14][1] = -c3e * 2.0 * y * z;
  dY[14][2] = c3e * (x * x - y * y);
  /* Y15 = -c3a (x^3 - 3 x y^2) */
  dY[15][0] = -c3a * (3.0 * x * x - 3.0 * y * y);
  dY[15][1] = -c3a * (-6.0 * x * y);
}

/* exported for the basis pin (Gram matrix under quadrature) */
void or_sh_basis(int deg, double x, double y, double z, double* Y) { sh_basis(deg, x, y, z, Y); }

/* ------------------------------------------------------------------------------------ */
/* rotation from a unit quaternion (w, x, y, z)                                          */
/* ------------------------------------------------------------------------------------ */
static void quat_to_rot(const double q[4], double R[3][3]) {
  const double w = q[0], x = q[1], y = q[2], z = q[3];
  R[0][0] = 1.0 - 2.0 * (y * y + z * z); R[0][1] = 2.0 * (x * y - w * z); R[0][2] = 2.0 * (x * z + w * y);
  R[1][0] = 2.0 * (x * y + w * z); R[1][1] = 1.0 - 2.0 * (x * x + z * z); R[1][2] = 2.0 * (y * z - w * x);
  R[2][0] = 2.0 * (x * z - w * y); R[2][1] = 2.0 * (y * z + w * x); R[2][2] = 1.0 - 2.0 * (x * x + y * y);
}

void or_quat_to_rot(const double* q, double* R9) {
  double R[3][3];
  quat_to_rot(q, R);
  for (int i = 0; i < 9; i++) R9[i] = R[i / 3][i % 3];
}

/* ------------------------------------------------------------------------------------ */
/* tile rect: the integer decision of binning, taken in float32                          */
/* ------------------------------------------------------------------------------------ */
/* clamp(f, 0, hi) for an integral float f, as an int (NaN -> 0). */
static int clamp_tile(float f, int hi) {
  if (!(f > 0.0f)) return 0;
  if (f > (float)hi) return hi;
  return (int)f;
}

/* rect [x0,x1) x [y0,y1) of tiles touched by the box of half-widths (rx, ry) around
 * (u, v): x0 = clamp(floor((u - rx)/16), 0, TX), x1 = clamp(floor((u + rx)/16) + 1, 0, TX),
 * the same in y.  u +- rx is one float32 add; the division by 16 is exact. */
static void tile_rect(float u, float v, int rx, int ry, int TX, int TY, int r[4]) {
  const float ulo = u - (float)rx, uhi = u + (float)rx;
  const float vlo = v - (float)ry, vhi = v + (float)ry;
  r[0] = clamp_tile(floorf(ulo * 0.0625f), TX);
  r[1] = clamp_tile(floorf(uhi * 0.0625f) + 1.0f, TX);
  r[2] = clamp_tile(floorf(vlo * 0.0625f), TY);
  r[3] = clamp_tile(floorf(vhi * 0.0625f) + 1.0f, TY);
}

/* ------------------------------------------------------------------------------------ */
/* forward of the per-Gaussian preprocess, shared by the forward and backward oracles     */
/* ------------------------------------------------------------------------------------ */
typedef struct {
  int visible;
  double s[3], o, qn[4], qlen, Rq[3][3], M[3][3], Sigma[3][3];
  double p[3];              /* camera-space position */
  double xc, yc;            /* clamped x/z, y/z */
  int xclamp, yclamp;       /* 1 when the guard-band clamp is active */
  double J[2][3], V[3][3], S2[2][2], det, Q[2][2];
  double u, v;
  int rx, ry, tiles;
  double dir[3], dist;      /* view direction mu - centre, normalised; |mu - centre| */
  double Y[16];
  double raw[3], rgb[3];
} fwd_t;

static void preprocess_one(const double* params, int64_t ld, int64_t i, int deg, const cam_t* k,
                           fwd_t* F) {
  memset(F, 0, sizeof(*F));
  double mu[3], l[3], q[4], a;
  for (int j = 0; j < 3; j++) mu[j] = params[(0 + j) * ld + i];
  for (int j = 0; j < 3; j++) l[j] = params[(3 + j) * ld + i];
  for (int j = 0; j < 4; j++) q[j] = params[(6 + j) * ld + i];
  a = params[10 * ld + i];
  for (int j = 0; j < 3; j++) if (!isfinite(mu[j]) || !isfinite(l[j])) return;
  for (int j = 0; j < 4; j++) if (!isfinite(q[j])) return;
  if (!isfinite(a)) return;

  /* activations: s = exp(l), o = sigmoid(a), q / |q| */
  for (int j = 0; j < 3; j++) F->s[j] = exp(l[j]);
  F->o = 1.0 / (1.0 + exp(-a));
  F->qlen = sqrt(q[0] * q[0] + q[1] * q[1] + q[2] * q[2] + q[3] * q[3]);
  if (!(F->qlen > 0.0) || !isfinite(F->qlen)) return;
  for (int j = 0; j < 4; j++) F->qn[j] = q[j] / F->qlen;

  /* covariance Sigma = M M^T with M = R(q) diag(s) */
  quat_to_rot(F->qn, F->Rq);
  for (int r = 0; r < 3; r++)
    for (int c = 0; c < 3; c++) F->M[r][c] = F->Rq[r][c] * F->s[c];
  for (int r = 0; r < 3; r++)
    for (int c = 0; c < 3; c++) {
      double acc = 0.0;
      for (int j = 0; j < 3; j++) acc += F->M[r][j] * F->M[c][j];
      F->Sigma[r][c] = acc;
    }

  /* camera transform p = Rc mu + t; near cull */
  for (int r = 0; r < 3; r++) {
    double acc = k->t[r];
    for (int j = 0; j < 3; j++) acc += k->Rc[r][j] * mu[j];
    F->p[r] = acc;
  }
  const double x = F->p[0], y = F->p[1], z = F->p[2];
  if (!isfinite(x) || !isfinite(y) || !isfinite(z)) return;
  if (!(z > k->near_plane)) return;

  /* pinhole projection */
  F->u = k->fx * x / z + k->cx;
  F->v = k->fy * y / z + k->cy;

  /* EWA: J at the guard-band clamped position, V = Rc Sigma Rc^T, S2 = J V J^T + 0.3 I */
  const double limx = GUARD * (0.5 * k->W) / k->fx, limy = GUARD * (0.5 * k->H) / k->fy;
  double tx = x / z, ty = y / z;
  F->xclamp = (tx < -limx || tx > limx);
  F->yclamp = (ty < -limy || ty > limy);
  F->xc = tx < -limx ? -limx : (tx > limx ? limx : tx);
  F->yc = ty < -limy ? -limy : (ty > limy ? limy : ty);
  F->J[0][0] = k->fx / z; F->J[0][1] = 0.0; F->J[0][2] = -k->fx * F->xc / z;
  F->J[1][0] = 0.0; F->J[1][1] = k->fy / z; F->J[1][2] = -k->fy * F->yc / z;
  double RS[3][3];
  for (int r = 0; r < 3; r++)
    for (int c = 0; c < 3; c++) {
      double acc = 0.0;
      for (int j = 0; j < 3; j++) acc += k->Rc[r][j] * F->Sigma[j][c];
      RS[r][c] = acc;
    }
  for (int r = 0; r < 3; r++)
    for (int c = 0; c < 3; c++) {
      double acc = 0.0;
      for (int j = 0; j < 3; j++) acc += RS[r][j] * k->Rc[c][j];
      F->V[r][c] = acc;
    }
  double JV[2][3];
  for (int r = 0; r < 2; r++)
    for (int c = 0; c < 3; c++) {
      double acc = 0.0;
      for (int j = 0; j < 3; j++) acc += F->J[r][j] * F->V[j][c];
      JV[r][c] = acc;
    }
  for (int r = 0; r < 2; r++)
    for (int c = 0; c < 2; c++) {
      double acc = 0.0;
      for (int j = 0; j < 3; j++) acc += JV[r][j] * F->J[c][j];
      F->S2[r][c] = acc + (r == c ? DILATION : 0.0);
    }

  /* conic = inverse of S2; cull degenerate */
  F->det = F->S2[0][0] * F->S2[1][1] - F->S2[0][1] * F->S2[0][1];
  if (!(F->det > 0.0) || !isfinite(F->det)) return;
  F->Q[0][0] = F->S2[1][1] / F->det;
  F->Q[0][1] = F->Q[1][0] = -F->S2[0][1] / F->det;
  F->Q[1][1] = F->S2[0][0] / F->det;

  /* per-axis 3-sigma radii, decided in float32 */
  F->rx = (int)ceilf(3.0f * sqrtf((float)F->S2[0][0]));
  F->ry = (int)ceilf(3.0f * sqrtf((float)F->S2[1][1]));
  int rect[4];
  tile_rect((float)F->u, (float)F->v, F->rx, F->ry, k->TX, k->TY, rect);
  F->tiles = (rect[1] - rect[0]) * (rect[3] - rect[2]);
  if (rect[1] <= rect[0] || rect[3] <= rect[2]) F->tiles = 0;
  if (F->tiles == 0) return;

  /* SH colour along the view direction, +0.5 offset, clamped at 0 */
  double dv[3];
  for (int j = 0; j < 3; j++) dv[j] = mu[j] - k->centre[j];
  F->dist = sqrt(dv[0] * dv[0] + dv[1] * dv[1] + dv[2] * dv[2]);
  for (int j = 0; j < 3; j++) F->dir[j] = dv[j] / F->dist;
  sh_basis(deg, F->dir[0], F->dir[1], F->dir[2], F->Y);
  const int nb = (deg + 1) * (deg + 1);
  for (int ch = 0; ch < 3; ch++) {
    double acc = 0.5;
    for (int kk = 0; kk < nb; kk++) acc += F->Y[kk] * params[(11 + 3 * kk + ch) * ld + i];
    F->raw[ch] = acc;
    F->rgb[ch] = acc > 0.0 ? acc : 0.0;
  }
  F->visible = 1;
}

/* gs preprocess (forward).  proj[10][n], radii[2][n], tiles[n]. */
int or_preprocess(int64_t n, int deg, const double* params, const double* camv, int W, int H,
                  double* proj, int32_t* radii, uint32_t* tiles) {
  cam_t k;
  load_cam(camv, W, H, &k);
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; i++) {
    fwd_t F;
    preprocess_one(params, n, i, deg, &k, &F);
    for (int f = 0; f < PRJ_FIELDS; f++) proj[f * n + i] = 0.0;
    radii[i] = radii[n + i] = 0;
    tiles[i] = 0;
    if (!F.visible) continue;
    proj[PRJ_U * n + i] = F.u;
    proj[PRJ_V * n + i] = F.v;
    proj[PRJ_DEPTH * n + i] = F.p[2];
    proj[PRJ_OPAC * n + i] = F.o;
    proj[PRJ_A * n + i] = F.Q[0][0];
    proj[PRJ_B * n + i] = F.Q[0][1];
    proj[PRJ_C * n + i] = F.Q[1][1];
    for (int ch = 0; ch < 3; ch++) proj[(PRJ_R + ch) * n + i] = F.rgb[ch];
    radii[i] = F.rx;
    radii[n + i] = F.ry;
    tiles[i] = (uint32_t)F.tiles;
  }
  return 0;
}

/* Diagnostics for borderline detection in the preprocess parity check:
 * out[0][i] = 3 sqrt(S2_00), out[1][i] = 3 sqrt(S2_11), out[2][i] = min |raw rgb| over
 * channels (distance of the colour clamp from switching).  Zero for culled. */
int or_preprocess_margins(int64_t n, int deg, const double* params, const double* camv, int W,
                          int H, double* out) {
  cam_t k;
  load_cam(camv, W, H, &k);
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; i++) {
    fwd_t F;
    preprocess_one(params, n, i, deg, &k, &F);
    out[i] = out[n + i] = out[2 * n + i] = 0.0;
    if (!F.visible) continue;
    out[i] = 3.0 * sqrt(F.S2[0][0]);
    out[n + i] = 3.0 * sqrt(F.S2[1][1]);
    double m = fabs(F.raw[0]);
    if (fabs(F.raw[1]) < m) m = fabs(F.raw[1]);
    if (fabs(F.raw[2]) < m) m = fabs(F.raw[2]);
    out[2 * n + i] = m;
  }
  return 0;
}

/* ------------------------------------------------------------------------------------ */
/* binning, stable sort, tile ranges                                                     */
/* ------------------------------------------------------------------------------------ */
static uint32_t float_bits(float f) {
  uint32_t b;
  memcpy(&b, &f, 4);
  return b;
}

/* Number of intersections for a projected set (u, v, depth read as float32). */
int64_t or_count_intersections(int64_t n, const double* proj, const int32_t* radii, int W, int H) {
  const int TX = (W + TILE - 1) / TILE, TY = (H + TILE - 1) / TILE;
  int64_t K = 0;
  for (int64_t i = 0; i < n; i++) {
    if (radii[i] == 0 || radii[n + i] == 0) continue;
    int r[4];
    tile_rect((float)proj[PRJ_U * n + i], (float)proj[PRJ_V * n + i], radii[i], radii[n + i], TX, TY, r);
    if (r[1] > r[0] && r[3] > r[2]) K += (int64_t)(r[1] - r[0]) * (r[3] - r[2]);
  }
  return K;
}

/* Tile rect [x0, x1) x [y0, y1) of every Gaussian (rect[0..3][n] = x0, x1, y0, y1; all 0 for
 * a culled one), the binning decision above (u, v read as float32). */
void or_tile_rects(int64_t n, const double* proj, const int32_t* radii, int W, int H, int32_t* rect) {
  const int TX = (W + TILE - 1) / TILE, TY = (H + TILE - 1) / TILE;
  for (int64_t i = 0; i < n; i++) {
    int r[4] = {0, 0, 0, 0};
    if (radii[i] != 0 && radii[n + i] != 0)
      tile_rect((float)proj[PRJ_U * n + i], (float)proj[PRJ_V * n + i], radii[i], radii[n + i], TX, TY, r);
    for (int j = 0; j < 4; j++) rect[j * n + i] = r[j];
  }
}

/* Stable bottom-up merge sort of (key, val) pairs by key. */
static void merge_sort_stable(uint64_t* key, uint32_t* val, int64_t K) {
  uint64_t* k2 = (uint64_t*)malloc((size_t)(K > 0 ? K : 1) * sizeof(uint64_t));
  uint32_t* v2 = (uint32_t*)malloc((size_t)(K > 0 ? K : 1) * sizeof(uint32_t));
  uint64_t *ks = key, *kd = k2;
  uint32_t *vs = val, *vd = v2;
  for (int64_t width = 1; width < K; width *= 2) {
    for (int64_t lo = 0; lo < K; lo += 2 * width) {
      int64_t mid = lo + width < K ? lo + width : K;
      int64_t hi = lo + 2 * width < K ? lo + 2 * width : K;
      int64_t a = lo, b = mid, o = lo;
      while (a < mid && b < hi) {
        if (ks[b] < ks[a]) { kd[o] = ks[b]; vd[o++] = vs[b++]; }  /* equal keys: left first */
        else { kd[o] = ks[a]; vd[o++] = vs[a++]; }
      }
      while (a < mid) { kd[o] = ks[a]; vd[o++] = vs[a++]; }
      while (b < hi) { kd[o] = ks[b]; vd[o++] = vs[b++]; }
    }
    uint64_t* tk = ks; ks = kd; kd = tk;
    uint32_t* tv = vs; vs = vd; vd = tv;
  }
  if (ks != key) {
    memcpy(key, ks, (size_t)K * sizeof(uint64_t));
    memcpy(val, vs, (size_t)K * sizeof(uint32_t));
  }
  free(k2);
  free(v2);
}

/* Keys ((ty*TX + tx) << 32 | bits(depth)), vals = Gaussian index, emitted per visible
 * Gaussian in increasing index and per tile of its rect in row-major order, then sorted
 * stably by key.  keys/vals must hold K entries (or_count_intersections). */
int64_t or_bin_sort(int64_t n, const double* proj, const int32_t* radii, int W, int H,
                    uint64_t* keys, uint32_t* vals) {
  const int TX = (W + TILE - 1) / TILE, TY = (H + TILE - 1) / TILE;
  int64_t slot = 0;
  for (int64_t i = 0; i < n; i++) {
    if (radii[i] == 0 || radii[n + i] == 0) continue;
    int r[4];
    tile_rect((float)proj[PRJ_U * n + i], (float)proj[PRJ_V * n + i], radii[i], radii[n + i], TX, TY, r);
    const uint64_t db = float_bits((float)proj[PRJ_DEPTH * n + i]);
    for (int ty = r[2]; ty < r[3]; ty++)
      for (int tx = r[0]; tx < r[1]; tx++) {
        keys[slot] = ((uint64_t)(ty * TX + tx) << 32) | db;
        vals[slot] = (uint32_t)i;
        slot++;
      }
  }
  merge_sort_stable(keys, vals, slot);
  return slot;
}

/* ranges[2*t] = first index with tile t, ranges[2*t+1] = one past the last; (0,0) if none. */
int or_ranges(int64_t K, const uint64_t* keys, int T, uint32_t* ranges) {
  for (int t = 0; t < 2 * T; t++) ranges[t] = 0;
  for (int64_t j = 0; j < K; j++) {
    const uint32_t t = (uint32_t)(keys[j] >> 32);
    if (j == 0 || (uint32_t)(keys[j - 1] >> 32) != t) ranges[2 * t] = (uint32_t)j;
    if (j == K - 1 || (uint32_t)(keys[j + 1] >> 32) != t) ranges[2 * t + 1] = (uint32_t)(j + 1);
  }
  return 0;
}

/* ------------------------------------------------------------------------------------ */
/* forward blend of one pixel                                                            */
/* ------------------------------------------------------------------------------------ */
/* Decision codes per examined entry (for the frozen-structure gradient checks). */
#define DEC_SKIP 0
#define DEC_BLEND 1
#define DEC_BLEND_CLAMPED 2
#define DEC_STOP 3
#define DEC_NONE 4 /* not examined (after termination) */

typedef struct {
  int64_t gi;          /* Gaussian index */
  double alpha, G, dx, dy, T_before;
  int clamped;
} contrib_t;

typedef struct {
  double margin_alpha;  /* relative margin around 1/255 */
  double margin_T;      /* relative margin around 1e-4 */
  double margin_power;  /* absolute margin above 0 */
} margins_t;

/* A running hash of the branch sequence a pixel's walk takes (FNV-1a over 64-bit words): the
 * index of every composited entry in order, then the index of the entry that stopped the walk
 * (flagged by the top bit) or nothing when the list ran out.  Two walks hash equal exactly when
 * (up to hash collisions) they composited the same Gaussians in the same order and stopped at the
 * same one.  Instrumentation only: it takes no part in the blend. */
static uint64_t walk_hash(uint64_t h, uint64_t word) {
  for (int b = 0; b < 8; b++) {
    h ^= (word >> (8 * b)) & 0xffu;
    h *= 0x100000001b3ull;
  }
  return h;
}
#define WALK_HASH_SEED 0xcbf29ce484222325ull

/* Blends pixel (px, py) over the list vals[start..end).  Writes the colour, the final
 * transmittance and the 1-based positions of the last blended / last examined entry.  If
 * `out` is non-null the composited entries are appended to it (size >= end-start); if `hash`
 * is non-null it receives the walk's hash (walk_hash). */
static void blend_pixel(int px, int py, const double* proj, int64_t n, const uint32_t* vals,
                        uint32_t start, uint32_t end, const double bg[3], double C[3],
                        double* T_final, uint32_t* last_contrib, uint32_t* n_examined,
                        contrib_t* out, int* n_out, const margins_t* mg, int* borderline,
                        int8_t* dec_out, const int8_t* dec_in, uint64_t* hash) {
  uint64_t h = WALK_HASH_SEED;
  double T = 1.0;
  C[0] = C[1] = C[2] = 0.0;
  uint32_t last = 0, examined = end - start;
  int cnt = 0, flag = 0;
  const double pxc = px + 0.5, pyc = py + 0.5;
  for (uint32_t j = start; j < end; j++) {
    const int64_t i = vals[j];
    const double dx = pxc - proj[PRJ_U * n + i], dy = pyc - proj[PRJ_V * n + i];
    const double A = proj[PRJ_A * n + i], B = proj[PRJ_B * n + i], Cc = proj[PRJ_C * n + i];
    const double o = proj[PRJ_OPAC * n + i];
    const double power = -0.5 * (A * dx * dx + Cc * dy * dy) - B * dx * dy;
    const double G = exp(power);
    const double oG = o * G;
    int code;
    if (dec_in) {
      code = dec_in[j - start];
    } else {
      if ((float)power > 0.0f) code = DEC_SKIP;
      else if ((float)oG < ALPHA_MIN_F) code = DEC_SKIP;
      else {
        const int clamped = (float)oG > ALPHA_MAX_F;
        const double alpha = clamped ? ALPHA_MAX : oG;
        const double Tn = T * (1.0 - alpha);
        code = ((float)Tn < T_MIN_F) ? DEC_STOP : (clamped ? DEC_BLEND_CLAMPED : DEC_BLEND);
      }
    }
    if (mg) {
      if (power >= 0.0 && power <= mg->margin_power) flag = 1;
      if (fabs(oG - 1.0 / 255.0) <= mg->margin_alpha * (1.0 / 255.0)) flag = 1;
      if (code != DEC_SKIP) {
        const double alpha = code == DEC_BLEND_CLAMPED ? ALPHA_MAX : (oG > ALPHA_MAX ? ALPHA_MAX : oG);
        const double Tn = T * (1.0 - alpha);
        if (fabs(Tn - 1e-4) <= mg->margin_T * 1e-4) flag = 1;
      }
    }
    if (dec_out) dec_out[j - start] = (int8_t)code;
    if (code == DEC_SKIP) continue;
    if (code == DEC_STOP) {
      examined = j - start + 1;
      h = walk_hash(h, (uint64_t)i | 0x8000000000000000ull);
      break;
    }
    h = walk_hash(h, (uint64_t)i);
    const int clamped = code == DEC_BLEND_CLAMPED;
    const double alpha = clamped ? ALPHA_MAX : oG;
    for (int ch = 0; ch < 3; ch++) C[ch] += proj[(PRJ_R + ch) * n + i] * alpha * T;
    if (out) {
      out[cnt].gi = i; out[cnt].alpha = alpha; out[cnt].G = G; out[cnt].dx = dx; out[cnt].dy = dy;
      out[cnt].T_before = T; out[cnt].clamped = clamped;
    }
    cnt++;
    T = T * (1.0 - alpha);
    last = j - start + 1;
  }
  if (dec_out)
    for (uint32_t j = start + examined; j < end; j++) dec_out[j - start] = DEC_NONE;
  for (int ch = 0; ch < 3; ch++) C[ch] += T * bg[ch];
  *T_final = T;
  *last_contrib = last;
  *n_examined = examined;
  if (n_out) *n_out = cnt;
  if (borderline) *borderline = flag;
  if (hash) *hash = h;
}

/* Tiled forward render.  image [H][W][3], T_final [H][W], last_contrib [H][W],
 * n_examined [H][W], borderline [H][W] (uint8, nullable), n_blended [H][W] (nullable: the
 * entries composited into each pixel), walk [H][W] (nullable: each pixel's walk hash).  `dec`
 * (nullable) is a per-pixel array of decision codes with row stride `dec_stride`; with
 * `dec_mode` = 1 the codes are written, with 2 they are read instead of testing the thresholds. */
int or_render_forward(int W, int H, const double* bg, int64_t n, const double* proj,
                      const uint32_t* vals, const uint32_t* ranges, double* image, double* T_final,
                      uint32_t* last_contrib, uint32_t* n_examined, uint8_t* borderline,
                      uint32_t* n_blended, const double* margins, int8_t* dec, int64_t dec_stride,
                      int dec_mode, uint64_t* walk) {
  const int TX = (W + TILE - 1) / TILE;
  margins_t mg = {1e-4, 1e-4, 1e-6};
  if (margins) { mg.margin_alpha = margins[0]; mg.margin_T = margins[1]; mg.margin_power = margins[2]; }
#pragma omp parallel for schedule(dynamic, 16)
  for (int64_t p = 0; p < (int64_t)W * H; p++) {
    const int px = (int)(p % W), py = (int)(p / W);
    const int t = (py / TILE) * TX + px / TILE;
    double C[3];
    int flag = 0, cnt = 0;
    int8_t* dp = dec ? dec + p * dec_stride : NULL;
    blend_pixel(px, py, proj, n, vals, ranges[2 * t], ranges[2 * t + 1], bg, C, &T_final[p],
                &last_contrib[p], &n_examined[p], NULL, &cnt, &mg, &flag,
                dec_mode == 1 ? dp : NULL, dec_mode == 2 ? dp : NULL, walk ? &walk[p] : NULL);
    for (int ch = 0; ch < 3; ch++) image[3 * p + ch] = C[ch];
    if (borderline) borderline[p] = (uint8_t)flag;
    if (n_blended) n_blended[p] = (uint32_t)cnt;
  }
  return 0;
}

/* Brute-force untiled render: every pixel gathers each visible Gaussian whose tile rect
 * contains the pixel's tile, orders them by (float32 depth bits, index) and blends. */
static int cmp_depth_index(const void* a, const void* b) {
  const uint64_t x = *(const uint64_t*)a, y = *(const uint64_t*)b;
  return x < y ? -1 : (x > y ? 1 : 0);
}

int or_render_bruteforce(int W, int H, const double* bg, int64_t n, const double* proj,
                         const int32_t* radii, double* image, double* T_final,
                         uint32_t* last_contrib, uint32_t* n_examined) {
  const int TX = (W + TILE - 1) / TILE, TY = (H + TILE - 1) / TILE;
  int* rect = (int*)malloc((size_t)(n > 0 ? n : 1) * 4 * sizeof(int));
  for (int64_t i = 0; i < n; i++) {
    if (radii[i] == 0 || radii[n + i] == 0) { rect[4 * i] = rect[4 * i + 1] = 0; continue; }
    tile_rect((float)proj[PRJ_U * n + i], (float)proj[PRJ_V * n + i], radii[i], radii[n + i], TX, TY,
              &rect[4 * i]);
  }
  uint64_t* order = (uint64_t*)malloc((size_t)(n > 0 ? n : 1) * sizeof(uint64_t));
  uint32_t* list = (uint32_t*)malloc((size_t)(n > 0 ? n : 1) * sizeof(uint32_t));
  for (int64_t p = 0; p < (int64_t)W * H; p++) {
    const int px = (int)(p % W), py = (int)(p / W), tx = px / TILE, ty = py / TILE;
    int64_t m = 0;
    for (int64_t i = 0; i < n; i++) {
      const int* r = &rect[4 * i];
      if (r[1] <= r[0] || r[3] <= r[2]) continue;
      if (tx >= r[0] && tx < r[1] && ty >= r[2] && ty < r[3])
        order[m++] = ((uint64_t)float_bits((float)proj[PRJ_DEPTH * n + i]) << 32) | (uint64_t)i;
    }
    qsort(order, (size_t)m, sizeof(uint64_t), cmp_depth_index);
    for (int64_t j = 0; j < m; j++) list[j] = (uint32_t)(order[j] & 0xffffffffu);
    double C[3];
    blend_pixel(px, py, proj, n, list, 0, (uint32_t)m, bg, C, &T_final[p], &last_contrib[p],
                &n_examined[p], NULL, NULL, NULL, NULL, NULL, NULL, NULL);
    for (int ch = 0; ch < 3; ch++) image[3 * p + ch] = C[ch];
  }
  (void)TY;
  free(rect);
  free(order);
  free(list);
  return 0;
}

/* ------------------------------------------------------------------------------------ */
/* L1 loss                                                                               */
/* ------------------------------------------------------------------------------------ */
/* L = mean |I - I*| over all count = 3HW elements; dL/dI = sign(I - I*) / count. */
double or_loss_l1(int64_t count, const double* image, const double* target, double* dLdI) {
  double acc = 0.0;
  for (int64_t e = 0; e < count; e++) {
    const double d = image[e] - target[e];
    acc += fabs(d);
    dLdI[e] = (d > 0.0 ? 1.0 : (d < 0.0 ? -1.0 : 0.0)) / (double)count;
  }
  return acc / (double)count;
}

/* ------------------------------------------------------------------------------------ */
/* L1 + D-SSIM loss ([Scaling], the loss passage: a lambda-weighted combination of an L1   */
/* term and a D-SSIM term; step "Compute the loss locally": L1 and fused SSIM)            */
/* ------------------------------------------------------------------------------------ */
/* The pages print neither the formula nor its constants.  Reading taken: SSIM of Wang et
 * al. with an 11x11 Gaussian window of standard deviation 1.5 (normalised to sum 1),
 * C1 = 0.01^2 and C2 = 0.03^2 for a data range of 1, computed per colour channel over the
 * window positions that lie wholly inside the image (no padding), and averaged over
 * channels and positions; D-SSIM = 1 - SSIM and
 *     L = (1 - lambda) * mean |I - I*| + lambda * (1 - SSIM).
 * Per position p (top-left corner of its window) and channel:
 *     mu_x = sum_w x, mu_y = sum_w y, var_x = sum_w x^2 - mu_x^2, var_y likewise,
 *     cov = sum_w x y - mu_x mu_y,
 *     S = (2 mu_x mu_y + C1)(2 cov + C2) / ((mu_x^2 + mu_y^2 + C1)(var_x + var_y + C2)).
 * The gradient with respect to the rendered image x follows the chain rule through the
 * three window sums that depend on x (sum_w x, sum_w x^2, sum_w x y):
 *     dS/d(sum_w x)   = S (2 mu_y / A - 2 mu_y / B - 2 mu_x / C + 2 mu_x / D)
 *     dS/d(sum_w x^2) = -S / D
 *     dS/d(sum_w x y) = 2 S / B
 * with A, B, C, D the four factors above in order, and each window sum passes its partial
 * back to every pixel of its window with the window weight (times 1, 2x or y).
 * image, target, dLdI: [H][W][3].  parts (nullable) receives {mean L1, mean SSIM}.
 * Returns L, or NAN when the image is smaller than the window. */
#define SSIM_WIN 11
#define SSIM_SIGMA 1.5
#define SSIM_C1 (0.01 * 0.01)
#define SSIM_C2 (0.03 * 0.03)

double or_loss_l1_dssim(int W, int H, const double* image, const double* target, double lambda,
                        double* parts, double* dLdI) {
  if (W < SSIM_WIN || H < SSIM_WIN) return NAN;
  double g[SSIM_WIN], gsum = 0.0;
  for (int a = 0; a < SSIM_WIN; a++) {
    const double d = (double)(a - SSIM_WIN / 2);
    g[a] = exp(-d * d / (2.0 * SSIM_SIGMA * SSIM_SIGMA));
    gsum += g[a];
  }
  for (int a = 0; a < SSIM_WIN; a++) g[a] /= gsum;
  const int Wv = W - SSIM_WIN + 1, Hv = H - SSIM_WIN + 1;
  const int64_t nv = (int64_t)Wv * Hv, npx = (int64_t)W * H;
  /* per channel and valid position: dS/d(sum x), dS/d(sum x^2), dS/d(sum xy) */
  double* d_mu = (double*)malloc((size_t)(3 * nv) * sizeof(double));
  double* d_xx = (double*)malloc((size_t)(3 * nv) * sizeof(double));
  double* d_xy = (double*)malloc((size_t)(3 * nv) * sizeof(double));
  /* per-row sums, added in row order afterwards: the total does not depend on the threads */
  double* ssim_row = (double*)calloc((size_t)Hv, sizeof(double));
#pragma omp parallel for schedule(static)
  for (int r = 0; r < Hv; r++) {
    for (int s = 0; s < Wv; s++) {
      for (int c = 0; c < 3; c++) {
        double mx = 0.0, my = 0.0, exx = 0.0, eyy = 0.0, exy = 0.0;
        for (int a = 0; a < SSIM_WIN; a++)
          for (int b = 0; b < SSIM_WIN; b++) {
            const double w = g[a] * g[b];
            const int64_t e = ((int64_t)(r + a) * W + (s + b)) * 3 + c;
            const double x = image[e], y = target[e];
            mx += w * x;
            my += w * y;
            exx += w * x * x;
            eyy += w * y * y;
            exy += w * x * y;
          }
        const double vx = exx - mx * mx, vy = eyy - my * my, cxy = exy - mx * my;
        const double A = 2.0 * mx * my + SSIM_C1, B = 2.0 * cxy + SSIM_C2;
        const double C = mx * mx + my * my + SSIM_C1, D = vx + vy + SSIM_C2;
        const double S = (A * B) / (C * D);
        ssim_row[r] += S;
        const int64_t p = (int64_t)c * nv + (int64_t)r * Wv + s;
        d_mu[p] = S * (2.0 * my / A - 2.0 * my / B - 2.0 * mx / C + 2.0 * mx / D);
        d_xx[p] = -S / D;
        d_xy[p] = 2.0 * S / B;
      }
    }
  }
  double ssim_sum = 0.0;
  for (int r = 0; r < Hv; r++) ssim_sum += ssim_row[r];
  free(ssim_row);
  const double M = 3.0 * (double)nv;
  const double ssim = ssim_sum / M;
  double l1_sum = 0.0;
  for (int64_t e = 0; e < 3 * npx; e++) l1_sum += fabs(image[e] - target[e]);
  const double l1 = l1_sum / (3.0 * (double)npx);
#pragma omp parallel for schedule(static)
  for (int qr = 0; qr < H; qr++) {
    for (int qs = 0; qs < W; qs++) {
      for (int c = 0; c < 3; c++) {
        const int64_t e = ((int64_t)qr * W + qs) * 3 + c;
        const double x = image[e], y = target[e];
        double dS = 0.0; /* d(sum over positions and channels of S) / dx */
        for (int a = 0; a < SSIM_WIN; a++) {
          const int r = qr - a;
          if (r < 0 || r >= Hv) continue;
          for (int b = 0; b < SSIM_WIN; b++) {
            const int s = qs - b;
            if (s < 0 || s >= Wv) continue;
            const int64_t p = (int64_t)c * nv + (int64_t)r * Wv + s;
            dS += g[a] * g[b] * (d_mu[p] + 2.0 * x * d_xx[p] + y * d_xy[p]);
          }
        }
        const double d = x - y;
        const double sgn = d > 0.0 ? 1.0 : (d < 0.0 ? -1.0 : 0.0);
        dLdI[e] = (1.0 - lambda) * sgn / (3.0 * (double)npx) - lambda * dS / M;
      }
    }
  }
  free(d_mu);
  free(d_xx);
  free(d_xy);
  if (parts) {
    parts[0] = l1;
    parts[1] = ssim;
  }
  return (1.0 - lambda) * l1 + lambda * (1.0 - ssim);
}

/* ------------------------------------------------------------------------------------ */
/* backward blend: exact derivative of the branch the forward took                       */
/* ------------------------------------------------------------------------------------ */
/* grad2d [9][n] (u, v, A, B, C, opacity, r, g, b), accumulated in double over pixels in
 * raster order.  dLdI [H][W][3].  `dec` as in or_render_forward (mode 2 = frozen). */
int or_render_backward(int W, int H, const double* bg, int64_t n, const double* proj,
                       const uint32_t* vals, const uint32_t* ranges, const double* dLdI,
                       double* grad2d, const int8_t* dec, int64_t dec_stride) {
  const int TX = (W + TILE - 1) / TILE;
  for (int64_t e = 0; e < 9 * n; e++) grad2d[e] = 0.0;
  uint32_t maxlen = 0;
  const int T = TX * ((H + TILE - 1) / TILE);
  for (int t = 0; t < T; t++)
    if (ranges[2 * t + 1] - ranges[2 * t] > maxlen) maxlen = ranges[2 * t + 1] - ranges[2 * t];
  contrib_t* list = (contrib_t*)malloc((size_t)(maxlen > 0 ? maxlen : 1) * sizeof(contrib_t));
  double* suffix = (double*)malloc((size_t)(maxlen + 1) * sizeof(double));
  for (int64_t p = 0; p < (int64_t)W * H; p++) {
    const int px = (int)(p % W), py = (int)(p / W);
    const int t = (py / TILE) * TX + px / TILE;
    double C[3], Tf;
    uint32_t last, ex;
    int cnt = 0;
    blend_pixel(px, py, proj, n, vals, ranges[2 * t], ranges[2 * t + 1], bg, C, &Tf, &last, &ex,
                list, &cnt, NULL, NULL, NULL, dec ? dec + p * dec_stride : NULL, NULL);
    const double* g = &dLdI[3 * p];
    const double bgg = bg[0] * g[0] + bg[1] * g[1] + bg[2] * g[2];
    /* suffix[k] = sum_{j >= k} alpha_j T_j (rgb_j . g) */
    suffix[cnt] = 0.0;
    for (int k = cnt - 1; k >= 0; k--) {
      const int64_t i = list[k].gi;
      const double cg = proj[PRJ_R * n + i] * g[0] + proj[PRJ_G * n + i] * g[1] + proj[PRJ_BL * n + i] * g[2];
      suffix[k] = suffix[k + 1] + list[k].alpha * list[k].T_before * cg;
    }
    for (int k = 0; k < cnt; k++) {
      const int64_t i = list[k].gi;
      const double a = list[k].alpha, Tk = list[k].T_before;
      const double cg = proj[PRJ_R * n + i] * g[0] + proj[PRJ_G * n + i] * g[1] + proj[PRJ_BL * n + i] * g[2];
      for (int ch = 0; ch < 3; ch++) grad2d[(6 + ch) * n + i] += a * Tk * g[ch];
      const double dL_dalpha = Tk * cg - (suffix[k + 1] + Tf * bgg) / (1.0 - a);
      if (list[k].clamped) continue; /* alpha = 0.99 does not depend on o or power */
      const double o = proj[PRJ_OPAC * n + i], G = list[k].G;
      const double dL_dpower = o * G * dL_dalpha;
      grad2d[5 * n + i] += G * dL_dalpha;
      const double dx = list[k].dx, dy = list[k].dy;
      const double A = proj[PRJ_A * n + i], B = proj[PRJ_B * n + i], Cc = proj[PRJ_C * n + i];
      grad2d[2 * n + i] += -0.5 * dx * dx * dL_dpower;
      grad2d[3 * n + i] += -dx * dy * dL_dpower;
      grad2d[4 * n + i] += -0.5 * dy * dy * dL_dpower;
      grad2d[0 * n + i] += (A * dx + B * dy) * dL_dpower;
      grad2d[1 * n + i] += (B * dx + Cc * dy) * dL_dpower;
    }
  }
  free(list);
  free(suffix);
  return 0;
}

/* ------------------------------------------------------------------------------------ */
/* preprocess backward: exact chain rule through the per-Gaussian forward                 */
/* ------------------------------------------------------------------------------------ */
int or_preprocess_backward(int64_t n, int deg, const double* params, const double* camv, int W,
                           int H, const double* grad2d, double* grads) {
  cam_t k;
  load_cam(camv, W, H, &k);
  const int R = or_rows_for_degree(deg), nb = (deg + 1) * (deg + 1);
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; i++) {
    for (int r = 0; r < R; r++) grads[r * n + i] = 0.0;
    fwd_t F;
    preprocess_one(params, n, i, deg, &k, &F);
    if (!F.visible) continue;
    const double gu = grad2d[0 * n + i], gv = grad2d[1 * n + i];
    const double gA = grad2d[2 * n + i], gB = grad2d[3 * n + i], gC = grad2d[4 * n + i];
    const double go = grad2d[5 * n + i];
    const double grgb[3] = {grad2d[6 * n + i], grad2d[7 * n + i], grad2d[8 * n + i]};
    double gmu[3] = {0.0, 0.0, 0.0};

    /* opacity: o = sigmoid(a) */
    grads[10 * n + i] = F.o * (1.0 - F.o) * go;

    /* colour: rgb = max(0.5 + sum_k Y_k(dir) f_k, 0) */
    double gc[3];
    for (int ch = 0; ch < 3; ch++) gc[ch] = F.raw[ch] > 0.0 ? grgb[ch] : 0.0;
    for (int kk = 0; kk < nb; kk++)
      for (int ch = 0; ch < 3; ch++) grads[(11 + 3 * kk + ch) * n + i] = F.Y[kk] * gc[ch];
    double dY[16][3];
    sh_basis_grad(deg, F.dir[0], F.dir[1], F.dir[2], dY);
    double gdir[3] = {0.0, 0.0, 0.0};
    for (int kk = 0; kk < nb; kk++)
      for (int ch = 0; ch < 3; ch++) {
        const double f = params[(11 + 3 * kk + ch) * n + i];
        for (int j = 0; j < 3; j++) gdir[j] += gc[ch] * f * dY[kk][j];
      }
    const double dd = F.dir[0] * gdir[0] + F.dir[1] * gdir[1] + F.dir[2] * gdir[2];
    for (int j = 0; j < 3; j++) gmu[j] += (gdir[j] - F.dir[j] * dd) / F.dist;

    /* conic Q = S2^{-1}:  dL/dS2 = -Q G_Q Q with G_Q = [[gA, gB/2], [gB/2, gC]] */
    const double GQ[2][2] = {{gA, 0.5 * gB}, {0.5 * gB, gC}};
    double QG[2][2], G2[2][2];
    for (int r = 0; r < 2; r++)
      for (int c = 0; c < 2; c++) QG[r][c] = F.Q[r][0] * GQ[0][c] + F.Q[r][1] * GQ[1][c];
    for (int r = 0; r < 2; r++)
      for (int c = 0; c < 2; c++) G2[r][c] = -(QG[r][0] * F.Q[0][c] + QG[r][1] * F.Q[1][c]);

    /* S2 = J V J^T + 0.3 I:  dL/dV = J^T G2 J,  dL/dJ = 2 G2 J V */
    double GV[3][3], GJ[2][3], G2J[2][3];
    for (int r = 0; r < 2; r++)
      for (int c = 0; c < 3; c++) G2J[r][c] = G2[r][0] * F.J[0][c] + G2[r][1] * F.J[1][c];
    for (int r = 0; r < 3; r++)
      for (int c = 0; c < 3; c++) GV[r][c] = F.J[0][r] * G2J[0][c] + F.J[1][r] * G2J[1][c];
    for (int r = 0; r < 2; r++)
      for (int c = 0; c < 3; c++) {
        double acc = 0.0;
        for (int j = 0; j < 3; j++) acc += G2J[r][j] * F.V[j][c];
        GJ[r][c] = 2.0 * acc;
      }

    /* V = Rc Sigma Rc^T:  dL/dSigma = Rc^T GV Rc */
    double T1[3][3], GS[3][3];
    for (int r = 0; r < 3; r++)
      for (int c = 0; c < 3; c++) {
        double acc = 0.0;
        for (int j = 0; j < 3; j++) acc += k.Rc[j][r] * GV[j][c];
        T1[r][c] = acc;
      }
    for (int r = 0; r < 3; r++)
      for (int c = 0; c < 3; c++) {
        double acc = 0.0;
        for (int j = 0; j < 3; j++) acc += T1[r][j] * k.Rc[j][c];
        GS[r][c] = acc;
      }

    /* Sigma = M M^T:  dL/dM = (GS + GS^T) M */
    double GM[3][3];
    for (int r = 0; r < 3; r++)
      for (int c = 0; c < 3; c++) {
        double acc = 0.0;
        for (int j = 0; j < 3; j++) acc += (GS[r][j] + GS[j][r]) * F.M[j][c];
        GM[r][c] = acc;
      }

    /* M = R diag(s): dL/ds_j = sum_i GM_ij R_ij, dL/dR_ij = GM_ij s_j; s = exp(l) */
    double GR[3][3];
    for (int c = 0; c < 3; c++) {
      double acc = 0.0;
      for (int r = 0; r < 3; r++) {
        acc += GM[r][c] * F.Rq[r][c];
        GR[r][c] = GM[r][c] * F.s[c];
      }
      grads[(3 + c) * n + i] = F.s[c] * acc;
    }

    /* R(q) with q = (w, x, y, z) unit: partial derivatives of each entry */
    const double w = F.qn[0], x = F.qn[1], y = F.qn[2], z = F.qn[3];
    const double dRw[3][3] = {{0, -2 * z, 2 * y}, {2 * z, 0, -2 * x}, {-2 * y, 2 * x, 0}};
    const double dRx[3][3] = {{0, 2 * y, 2 * z}, {2 * y, -4 * x, -2 * w}, {2 * z, 2 * w, -4 * x}};
    const double dRy[3][3] = {{-4 * y, 2 * x, 2 * w}, {2 * x, 0, 2 * z}, {-2 * w, 2 * z, -4 * y}};
    const double dRz[3][3] = {{-4 * z, -2 * w, 2 * x}, {2 * w, -4 * z, 2 * y}, {2 * x, 2 * y, 0}};
    double gq[4] = {0, 0, 0, 0};
    for (int r = 0; r < 3; r++)
      for (int c = 0; c < 3; c++) {
        gq[0] += GR[r][c] * dRw[r][c];
        gq[1] += GR[r][c] * dRx[r][c];
        gq[2] += GR[r][c] * dRy[r][c];
        gq[3] += GR[r][c] * dRz[r][c];
      }
    /* q_hat = q / |q| */
    const double qd = F.qn[0] * gq[0] + F.qn[1] * gq[1] + F.qn[2] * gq[2] + F.qn[3] * gq[3];
    for (int j = 0; j < 4; j++) grads[(6 + j) * n + i] = (gq[j] - F.qn[j] * qd) / F.qlen;

    /* camera-space position: through (u, v) and through J */
    const double px = F.p[0], py = F.p[1], pz = F.p[2];
    double gp[3];
    gp[0] = gu * k.fx / pz;
    gp[1] = gv * k.fy / pz;
    gp[2] = -gu * k.fx * px / (pz * pz) - gv * k.fy * py / (pz * pz);
    /* J00 = fx/z, J11 = fy/z */
    gp[2] += GJ[0][0] * (-k.fx / (pz * pz)) + GJ[1][1] * (-k.fy / (pz * pz));
    /* J02 = -fx xc / z with xc = x/z unless clamped (then a constant) */
    if (!F.xclamp) {
      gp[0] += GJ[0][2] * (-k.fx / (pz * pz));
      gp[2] += GJ[0][2] * (2.0 * k.fx * px / (pz * pz * pz));
    } else {
      gp[2] += GJ[0][2] * (k.fx * F.xc / (pz * pz));
    }
    if (!F.yclamp) {
      gp[1] += GJ[1][2] * (-k.fy / (pz * pz));
      gp[2] += GJ[1][2] * (2.0 * k.fy * py / (pz * pz * pz));
    } else {
      gp[2] += GJ[1][2] * (k.fy * F.yc / (pz * pz));
    }
    /* p = Rc mu + t */
    for (int j = 0; j < 3; j++) gmu[j] += k.Rc[0][j] * gp[0] + k.Rc[1][j] * gp[1] + k.Rc[2][j] * gp[2];
    for (int j = 0; j < 3; j++) grads[j * n + i] = gmu[j];
  }
  return 0;
}

/* ------------------------------------------------------------------------------------ */
/* Adam (Kingma & Ba), dense, bias-corrected, in place                                    */
/* ------------------------------------------------------------------------------------ */
int or_adam(int64_t count, double* theta, const double* g, double* m, double* v, int t, double lr,
            double b1, double b2, double eps) {
  const double c1 = 1.0 - pow(b1, t), c2 = 1.0 - pow(b2, t);
  for (int64_t e = 0; e < count; e++) {
    m[e] = b1 * m[e] + (1.0 - b1) * g[e];
    v[e] = b2 * v[e] + (1.0 - b2) * g[e] * g[e];
    const double mh = m[e] / c1, vh = v[e] / c2;
    theta[e] -= lr * mh / (sqrt(vh) + eps);
  }
  return 0;
}

/* ------------------------------------------------------------------------------------ */
/* per-Gaussian intermediates for the pins (one Gaussian, its R parameters in `p`)        */
/* ------------------------------------------------------------------------------------ */
/* out: [0] visible, [1..3] s, [4] o, [5..13] R(q), [14..22] Sigma, [23..25] p_cam,
 * [26..31] J (2x3), [32..40] V, [41..44] S2, [45..48] Q, [49] u, [50] v, [51] rx, [52] ry,
 * [53] tiles, [54..56] dir, [57..59] raw rgb, [60..62] rgb */
int or_debug_gaussian(int deg, const double* p, const double* camv, int W, int H, double* out) {
  cam_t k;
  load_cam(camv, W, H, &k);
  fwd_t F;
  preprocess_one(p, 1, 0, deg, &k, &F);
  for (int e = 0; e < 63; e++) out[e] = 0.0;
  out[0] = F.visible;
  for (int j = 0; j < 3; j++) out[1 + j] = F.s[j];
  out[4] = F.o;
  for (int e = 0; e < 9; e++) out[5 + e] = F.Rq[e / 3][e % 3];
  for (int e = 0; e < 9; e++) out[14 + e] = F.Sigma[e / 3][e % 3];
  for (int j = 0; j < 3; j++) out[23 + j] = F.p[j];
  for (int e = 0; e < 6; e++) out[26 + e] = F.J[e / 3][e % 3];
  for (int e = 0; e < 9; e++) out[32 + e] = F.V[e / 3][e % 3];
  for (int e = 0; e < 4; e++) out[41 + e] = F.S2[e / 2][e % 2];
  for (int e = 0; e < 4; e++) out[45 + e] = F.Q[e / 2][e % 2];
  out[49] = F.u; out[50] = F.v; out[51] = F.rx; out[52] = F.ry; out[53] = F.tiles;
  for (int j = 0; j < 3; j++) { out[54 + j] = F.dir[j]; out[57 + j] = F.raw[j]; out[60 + j] = F.rgb[j]; }
  return 0;
}
