/*
 * _kvstore_py: the CPython binding of libkvstore (include/kvstore.h).
 *
 * Argument marshalling only: every function takes Python ints (pointers as
 * ints, None for NULL), calls the C function of the same name and returns its
 * status.  Functions use the vectorcall convention (METH_FASTCALL), so a call
 * converts its integers directly with no argument tuple; the GIL is released
 * around each library call, so threads can issue stores concurrently.
 */
#define PY_SSIZE_T_CLEAN
#include <Python.h>

#include <stdint.h>

#include "kvstore.h"

/* A device or host pointer from a Python int, or NULL from None. */
static int to_ptr(PyObject* o, void** out) {
  if (o == Py_None) {
    *out = NULL;
    return 1;
  }
  void* p = PyLong_AsVoidPtr(o);
  if (p == NULL && PyErr_Occurred()) return 0;
  *out = p;
  return 1;
}

static int to_i64(PyObject* o, int64_t* out) {
  long long v = PyLong_AsLongLong(o);
  if (v == -1 && PyErr_Occurred()) return 0;
  *out = (int64_t)v;
  return 1;
}

static int to_int(PyObject* o, int* out) {
  long v = PyLong_AsLong(o);
  if (v == -1 && PyErr_Occurred()) return 0;
  if (v < INT32_MIN || v > INT32_MAX) {
    PyErr_SetString(PyExc_OverflowError, "value does not fit in a C int");
    return 0;
  }
  *out = (int)v;
  return 1;
}

static int to_u32(PyObject* o, uint32_t* out) {
  unsigned long long v = PyLong_AsUnsignedLongLong(o);
  if (v == (unsigned long long)-1 && PyErr_Occurred()) return 0;
  if (v > UINT32_MAX) {
    PyErr_SetString(PyExc_OverflowError, "batch does not fit in 32 bits");
    return 0;
  }
  *out = (uint32_t)v;
  return 1;
}

/* The stream argument: optional, None or 0 for the null stream. */
static int stream_arg(PyObject* const* args, Py_ssize_t nargs, Py_ssize_t i, hipStream_t* s) {
  void* p = NULL;
  if (nargs > i && !to_ptr(args[i], &p)) return 0;
  *s = (hipStream_t)p;
  return 1;
}

static int check_nargs(const char* name, Py_ssize_t nargs, Py_ssize_t need) {
  if (nargs == need || nargs == need + 1) return 1;
  PyErr_Format(PyExc_TypeError, "%s takes %zd arguments (+ optional stream), got %zd", name,
               need, nargs);
  return 0;
}

static PyObject* py_kvstore_copy(PyObject* self, PyObject* const* a, Py_ssize_t n) {
  (void)self;
  void *k, *v, *kc, *vc, *ix;
  int idx_dtype;
  int64_t idx_stride, row, ks, vs, cs, limit;
  uint32_t batch;
  hipStream_t s;
  if (!check_nargs("kvstore_copy", n, 13) || !to_ptr(a[0], &k) || !to_ptr(a[1], &v) ||
      !to_ptr(a[2], &kc) || !to_ptr(a[3], &vc) || !to_ptr(a[4], &ix) ||
      !to_int(a[5], &idx_dtype) || !to_i64(a[6], &idx_stride) || !to_i64(a[7], &row) ||
      !to_i64(a[8], &ks) || !to_i64(a[9], &vs) || !to_i64(a[10], &cs) ||
      !to_u32(a[11], &batch) || !to_i64(a[12], &limit) || !stream_arg(a, n, 13, &s))
    return NULL;
  int st;
  Py_BEGIN_ALLOW_THREADS
  st = kvstore_copy(k, v, kc, vc, ix, idx_dtype, idx_stride, row, ks, vs, cs, batch, limit, s);
  Py_END_ALLOW_THREADS
  return PyLong_FromLong(st);
}

/* Arguments shared by the three FP8 stores, up to and including page_size. */
typedef struct {
  void *k, *v, *kc, *vc, *ix;
  int idx_dtype, src_dtype, heads, dim;
  int64_t idx_stride, kt, kh, vt, vh, kcp, kco, kch, vcp, vco, vch, limit, page;
  uint32_t batch;
} Fp8Args;

/* a[0..19] plus batch, size_limit and page_size at b, b + 1, b + 2. */
static int fp8_args(PyObject* const* a, Py_ssize_t b, Fp8Args* f) {
  return to_ptr(a[0], &f->k) && to_ptr(a[1], &f->v) && to_ptr(a[2], &f->kc) &&
         to_ptr(a[3], &f->vc) && to_ptr(a[4], &f->ix) && to_int(a[5], &f->idx_dtype) &&
         to_i64(a[6], &f->idx_stride) && to_int(a[7], &f->src_dtype) &&
         to_int(a[8], &f->heads) && to_int(a[9], &f->dim) && to_i64(a[10], &f->kt) &&
         to_i64(a[11], &f->kh) && to_i64(a[12], &f->vt) && to_i64(a[13], &f->vh) &&
         to_i64(a[14], &f->kcp) && to_i64(a[15], &f->kco) && to_i64(a[16], &f->kch) &&
         to_i64(a[17], &f->vcp) && to_i64(a[18], &f->vco) && to_i64(a[19], &f->vch) &&
         to_u32(a[b], &f->batch) && to_i64(a[b + 1], &f->limit) && to_i64(a[b + 2], &f->page);
}

static PyObject* fp8_static(PyObject* const* a, Py_ssize_t n, int e5m2) {
  const char* name = e5m2 ? "kvstore_fp8_paged_e5m2" : "kvstore_fp8_paged";
  Fp8Args f;
  void *ik, *iv;
  hipStream_t s;
  if (!check_nargs(name, n, 25) || !fp8_args(a, 20, &f) || !to_ptr(a[23], &ik) ||
      !to_ptr(a[24], &iv) || !stream_arg(a, n, 25, &s))
    return NULL;
  int st;
  Py_BEGIN_ALLOW_THREADS
  st = (e5m2 ? kvstore_fp8_paged_e5m2 : kvstore_fp8_paged)(
      f.k, f.v, f.kc, f.vc, f.ix, f.idx_dtype, f.idx_stride, f.src_dtype, f.heads, f.dim, f.kt,
      f.kh, f.vt, f.vh, f.kcp, f.kco, f.kch, f.vcp, f.vco, f.vch, f.batch, f.limit, f.page,
      (const float*)ik, (const float*)iv, s);
  Py_END_ALLOW_THREADS
  return PyLong_FromLong(st);
}

static PyObject* py_kvstore_fp8_paged(PyObject* self, PyObject* const* a, Py_ssize_t n) {
  (void)self;
  return fp8_static(a, n, 0);
}

static PyObject* py_kvstore_fp8_paged_e5m2(PyObject* self, PyObject* const* a, Py_ssize_t n) {
  (void)self;
  return fp8_static(a, n, 1);
}

static PyObject* py_kvstore_fp8_paged_dynamic(PyObject* self, PyObject* const* a, Py_ssize_t n) {
  (void)self;
  Fp8Args f;
  void *ksc, *vsc;
  int gran;
  int64_t ksp, kso, ksh, vsp, vso, vsh;
  hipStream_t s;
  if (!check_nargs("kvstore_fp8_paged_dynamic", n, 32) || !fp8_args(a, 29, &f) ||
      !to_ptr(a[20], &ksc) || !to_ptr(a[21], &vsc) || !to_int(a[22], &gran) ||
      !to_i64(a[23], &ksp) || !to_i64(a[24], &kso) || !to_i64(a[25], &ksh) ||
      !to_i64(a[26], &vsp) || !to_i64(a[27], &vso) || !to_i64(a[28], &vsh) ||
      !stream_arg(a, n, 32, &s))
    return NULL;
  int st;
  Py_BEGIN_ALLOW_THREADS
  st = kvstore_fp8_paged_dynamic(f.k, f.v, f.kc, f.vc, f.ix, f.idx_dtype, f.idx_stride,
                                 f.src_dtype, f.heads, f.dim, f.kt, f.kh, f.vt, f.vh, f.kcp,
                                 f.kco, f.kch, f.vcp, f.vco, f.vch, (float*)ksc, (float*)vsc,
                                 gran, ksp, kso, ksh, vsp, vso, vsh, f.batch, f.limit, f.page, s);
  Py_END_ALLOW_THREADS
  return PyLong_FromLong(st);
}

static PyObject* py_kvstore_check_error(PyObject* self, PyObject* const* a, Py_ssize_t n) {
  (void)self;
  hipStream_t s;
  if (n > 1) {
    PyErr_SetString(PyExc_TypeError, "kvstore_check_error takes an optional stream");
    return NULL;
  }
  if (!stream_arg(a, n, 0, &s)) return NULL;
  int64_t first_bad = 0;
  uint64_t count = 0;
  int st;
  Py_BEGIN_ALLOW_THREADS
  st = kvstore_check_error(s, &first_bad, &count);
  Py_END_ALLOW_THREADS
  return Py_BuildValue("(iLK)", st, (long long)first_bad, (unsigned long long)count);
}

static PyObject* py_kvstore_take_error(PyObject* self, PyObject* const* a, Py_ssize_t n) {
  (void)self;
  void* out;
  hipStream_t s;
  if (!check_nargs("kvstore_take_error", n, 1) || !to_ptr(a[0], &out) ||
      !stream_arg(a, n, 1, &s))
    return NULL;
  int st;
  Py_BEGIN_ALLOW_THREADS
  st = kvstore_take_error((int64_t*)out, s);
  Py_END_ALLOW_THREADS
  return PyLong_FromLong(st);
}

static PyObject* py_kvstore_strerror(PyObject* self, PyObject* const* a, Py_ssize_t n) {
  (void)self;
  int status;
  if (n != 1) {
    PyErr_SetString(PyExc_TypeError, "kvstore_strerror takes one status");
    return NULL;
  }
  if (!to_int(a[0], &status)) return NULL;
  return PyUnicode_FromString(kvstore_strerror(status));
}

#define FASTCALL(f) ((PyCFunction)(void (*)(void))(f))

static PyMethodDef methods[] = {
    {"kvstore_copy", FASTCALL(py_kvstore_copy), METH_FASTCALL, "See include/kvstore.h."},
    {"kvstore_fp8_paged", FASTCALL(py_kvstore_fp8_paged), METH_FASTCALL,
     "See include/kvstore.h."},
    {"kvstore_fp8_paged_e5m2", FASTCALL(py_kvstore_fp8_paged_e5m2), METH_FASTCALL,
     "See include/kvstore.h."},
    {"kvstore_fp8_paged_dynamic", FASTCALL(py_kvstore_fp8_paged_dynamic), METH_FASTCALL,
     "See include/kvstore.h."},
    {"kvstore_check_error", FASTCALL(py_kvstore_check_error), METH_FASTCALL,
     "Returns (status, first_bad_token, bad_count)."},
    {"kvstore_take_error", FASTCALL(py_kvstore_take_error), METH_FASTCALL,
     "See include/kvstore.h."},
    {"kvstore_strerror", FASTCALL(py_kvstore_strerror), METH_FASTCALL, "Status text."},
    {NULL, NULL, 0, NULL}};

static struct PyModuleDef module = {PyModuleDef_HEAD_INIT, "_kvstore_py",
                                    "CPython binding of libkvstore.", -1, methods,
                                    NULL, NULL, NULL, NULL};

PyMODINIT_FUNC PyInit__kvstore_py(void) { return PyModule_Create(&module); }
