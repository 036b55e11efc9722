/* _moe_fast: the per-call entry points of libmoe_a2a.so for Python, with
 * argument conversion done in C.  A decode step is two launches of a few
 * microseconds each, so the host cost of a call matters: converting seven
 * arguments through ctypes costs more than the launch itself.  Each function
 * takes the address of a moe_handle, device pointers as Python ints (None
 * for NULL), sizes as ints, and returns the library's int code unchanged;
 * the Python layer checks tensors and raises on a nonzero code.  Nothing is
 * computed here. */
#define PY_SSIZE_T_CLEAN
#include <Python.h>
#include <limits.h>

#include "moe_a2a.h"

static int ptr_arg(PyObject *o, void **out) {
    if (o == Py_None) {
        *out = NULL;
        return 0;
    }
    *out = PyLong_AsVoidPtr(o);
    return (*out == NULL && PyErr_Occurred()) ? -1 : 0;
}

static int i32_arg(PyObject *o, int32_t *out) {
    const long v = PyLong_AsLong(o);
    if (v == -1 && PyErr_Occurred()) return -1;
    if (v < INT32_MIN || v > INT32_MAX) {
        PyErr_SetString(PyExc_OverflowError, "argument does not fit int32");
        return -1;
    }
    *out = (int32_t)v;
    return 0;
}

static int want_args(Py_ssize_t nargs, Py_ssize_t n, const char *name) {
    if (nargs == n) return 0;
    PyErr_Format(PyExc_TypeError, "%s takes %zd arguments (%zd given)", name, n, nargs);
    return -1;
}

/* dispatch(handle, x, topk_ids, num_tokens, runtime_max_tokens_per_rank, workspace, stream) */
static PyObject *fast_dispatch(PyObject *self, PyObject *const *args, Py_ssize_t nargs) {
    void *h, *x, *ids, *ws, *stream;
    int32_t T, R;
    (void)self;
    if (want_args(nargs, 7, "dispatch") || ptr_arg(args[0], &h) || ptr_arg(args[1], &x) ||
        ptr_arg(args[2], &ids) || i32_arg(args[3], &T) || i32_arg(args[4], &R) ||
        ptr_arg(args[5], &ws) || ptr_arg(args[6], &stream))
        return NULL;
    return PyLong_FromLong(moe_dispatch((moe_handle *)h, (const uint16_t *)x, (const int32_t *)ids,
                                        T, R, (uint16_t *)ws, stream));
}

/* dispatch_fp8(handle, x, topk_ids, num_tokens, runtime_max_tokens_per_rank, workspace, scales, stream) */
static PyObject *fast_dispatch_fp8(PyObject *self, PyObject *const *args, Py_ssize_t nargs) {
    void *h, *x, *ids, *ws, *scales, *stream;
    int32_t T, R;
    (void)self;
    if (want_args(nargs, 8, "dispatch_fp8") || ptr_arg(args[0], &h) || ptr_arg(args[1], &x) ||
        ptr_arg(args[2], &ids) || i32_arg(args[3], &T) || i32_arg(args[4], &R) ||
        ptr_arg(args[5], &ws) || ptr_arg(args[6], &scales) || ptr_arg(args[7], &stream))
        return NULL;
    return PyLong_FromLong(moe_dispatch_fp8((moe_handle *)h, (const uint16_t *)x,
                                            (const int32_t *)ids, T, R, (uint8_t *)ws,
                                            (float *)scales, stream));
}

/* combine(handle, expert_out, topk_weights, weighted, out, stream) */
static PyObject *fast_combine(PyObject *self, PyObject *const *args, Py_ssize_t nargs) {
    void *h, *y, *w, *out, *stream;
    int32_t weighted;
    (void)self;
    if (want_args(nargs, 6, "combine") || ptr_arg(args[0], &h) || ptr_arg(args[1], &y) ||
        ptr_arg(args[2], &w) || i32_arg(args[3], &weighted) || ptr_arg(args[4], &out) ||
        ptr_arg(args[5], &stream))
        return NULL;
    return PyLong_FromLong(moe_combine((moe_handle *)h, (const uint16_t *)y, (const float *)w,
                                       weighted, (uint16_t *)out, stream));
}

/* combine_residual_rmsnorm(handle, expert_out, topk_weights, weighted, residual,
 *                          residual_out, gamma, eps, normed, stream) */
static PyObject *fast_combine_residual_rmsnorm(PyObject *self, PyObject *const *args,
                                               Py_ssize_t nargs) {
    void *h, *y, *w, *res, *res_out, *gamma, *normed, *stream;
    int32_t weighted;
    double eps;
    (void)self;
    if (want_args(nargs, 10, "combine_residual_rmsnorm") || ptr_arg(args[0], &h) ||
        ptr_arg(args[1], &y) || ptr_arg(args[2], &w) || i32_arg(args[3], &weighted) ||
        ptr_arg(args[4], &res) || ptr_arg(args[5], &res_out) || ptr_arg(args[6], &gamma))
        return NULL;
    eps = PyFloat_AsDouble(args[7]);
    if (eps == -1.0 && PyErr_Occurred()) return NULL;
    if (ptr_arg(args[8], &normed) || ptr_arg(args[9], &stream)) return NULL;
    return PyLong_FromLong(moe_combine_residual_rmsnorm(
        (moe_handle *)h, (const uint16_t *)y, (const float *)w, weighted, (const uint16_t *)res,
        (uint16_t *)res_out, (const uint16_t *)gamma, (float)eps, (uint16_t *)normed, stream));
}

/* route_counts(handle, topk_ids, num_tokens, stream) */
static PyObject *fast_route_counts(PyObject *self, PyObject *const *args, Py_ssize_t nargs) {
    void *h, *ids, *stream;
    int32_t T;
    (void)self;
    if (want_args(nargs, 4, "route_counts") || ptr_arg(args[0], &h) || ptr_arg(args[1], &ids) ||
        i32_arg(args[2], &T) || ptr_arg(args[3], &stream))
        return NULL;
    return PyLong_FromLong(moe_route_counts((moe_handle *)h, (const int32_t *)ids, T, stream));
}

/* partials_reduce(partials, num_partials, num_tokens, hidden, out, stream) */
static PyObject *fast_partials_reduce(PyObject *self, PyObject *const *args, Py_ssize_t nargs) {
    void *partials, *out, *stream;
    int32_t P, T, H;
    (void)self;
    if (want_args(nargs, 6, "partials_reduce") || ptr_arg(args[0], &partials) ||
        i32_arg(args[1], &P) || i32_arg(args[2], &T) || i32_arg(args[3], &H) ||
        ptr_arg(args[4], &out) || ptr_arg(args[5], &stream))
        return NULL;
    return PyLong_FromLong(moe_partials_reduce((const uint16_t *)partials, P, T, H,
                                               (uint16_t *)out, stream));
}

/* partials_reduce_residual_rmsnorm(partials, num_partials, num_tokens, hidden, residual,
 *                                  residual_out, gamma, eps, normed, stream) */
static PyObject *fast_partials_reduce_residual_rmsnorm(PyObject *self, PyObject *const *args,
                                                       Py_ssize_t nargs) {
    void *partials, *res, *res_out, *gamma, *normed, *stream;
    int32_t P, T, H;
    double eps;
    (void)self;
    if (want_args(nargs, 10, "partials_reduce_residual_rmsnorm") ||
        ptr_arg(args[0], &partials) || i32_arg(args[1], &P) || i32_arg(args[2], &T) ||
        i32_arg(args[3], &H) || ptr_arg(args[4], &res) || ptr_arg(args[5], &res_out) ||
        ptr_arg(args[6], &gamma))
        return NULL;
    eps = PyFloat_AsDouble(args[7]);
    if (eps == -1.0 && PyErr_Occurred()) return NULL;
    if (ptr_arg(args[8], &normed) || ptr_arg(args[9], &stream)) return NULL;
    return PyLong_FromLong(moe_partials_reduce_residual_rmsnorm(
        (const uint16_t *)partials, P, T, H, (const uint16_t *)res, (uint16_t *)res_out,
        (const uint16_t *)gamma, (float)eps, (uint16_t *)normed, stream));
}

static PyMethodDef methods[] = {
    {"dispatch", (PyCFunction)(void (*)(void))fast_dispatch, METH_FASTCALL, "moe_dispatch"},
    {"dispatch_fp8", (PyCFunction)(void (*)(void))fast_dispatch_fp8, METH_FASTCALL,
     "moe_dispatch_fp8"},
    {"combine", (PyCFunction)(void (*)(void))fast_combine, METH_FASTCALL, "moe_combine"},
    {"combine_residual_rmsnorm", (PyCFunction)(void (*)(void))fast_combine_residual_rmsnorm,
     METH_FASTCALL, "moe_combine_residual_rmsnorm"},
    {"route_counts", (PyCFunction)(void (*)(void))fast_route_counts, METH_FASTCALL,
     "moe_route_counts"},
    {"partials_reduce", (PyCFunction)(void (*)(void))fast_partials_reduce, METH_FASTCALL,
     "moe_partials_reduce"},
    {"partials_reduce_residual_rmsnorm",
     (PyCFunction)(void (*)(void))fast_partials_reduce_residual_rmsnorm, METH_FASTCALL,
     "moe_partials_reduce_residual_rmsnorm"},
    {NULL, NULL, 0, NULL},
};

static struct PyModuleDef module = {
    PyModuleDef_HEAD_INIT, "_moe_fast",
    "Per-call entry points of libmoe_a2a.so with argument conversion in C.", -1, methods,
    NULL, NULL, NULL, NULL,
};

PyMODINIT_FUNC PyInit__moe_fast(void) { return PyModule_Create(&module); }
