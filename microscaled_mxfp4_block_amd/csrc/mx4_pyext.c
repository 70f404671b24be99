/*
 * mx4_pyext.c -- CPython fast-call wrappers for the hot entry points of
 * libmx4.so.  Argument marshalling only: integers (device pointers, sizes, a
 * hipStream_t as an integer) in, the MX_* return code out.  The ctypes
 * binding covers every entry point; this module exists so that a Python
 * caller pays ~0.1 us instead of ~1-2 us of ctypes conversion per GEMM call.
 */
#define PY_SSIZE_T_CLEAN
#include <Python.h>
#include <stdint.h>

#include "../../include/mx4.h"

static int get_ptr(PyObject* o, void** out) {
    if (o == Py_None) {
        *out = NULL;
        return 0;
    }
    unsigned long long v = PyLong_AsUnsignedLongLong(o);
    if (v == (unsigned long long)-1 && PyErr_Occurred()) return -1;
    *out = (void*)(uintptr_t)v;
    return 0;
}

static int get_int(PyObject* o, int* out) {
    long v = PyLong_AsLong(o);
    if (v == -1 && PyErr_Occurred()) return -1;
    if (v < INT32_MIN || v > INT32_MAX) {
        PyErr_SetString(PyExc_OverflowError, "argument does not fit in a C int");
        return -1;
    }
    *out = (int)v;
    return 0;
}

static int get_size(PyObject* o, size_t* out) {
    unsigned long long v = PyLong_AsUnsignedLongLong(o);
    if (v == (unsigned long long)-1 && PyErr_Occurred()) return -1;
    *out = (size_t)v;
    return 0;
}

/* gemm(A, M, K, lda, packed, N, C, ldc, ws, ws_bytes, stream) -> rc */
static PyObject* py_gemm(PyObject* self, PyObject* const* a, Py_ssize_t n) {
    (void)self;
    if (n != 11) {
        PyErr_SetString(PyExc_TypeError, "gemm expects 11 arguments");
        return NULL;
    }
    void *A, *P, *C, *W, *S;
    int M, K, lda, N, ldc;
    size_t wsb;
    if (get_ptr(a[0], &A) || get_int(a[1], &M) || get_int(a[2], &K) || get_int(a[3], &lda) ||
        get_ptr(a[4], &P) || get_int(a[5], &N) || get_ptr(a[6], &C) || get_int(a[7], &ldc) ||
        get_ptr(a[8], &W) || get_size(a[9], &wsb) || get_ptr(a[10], &S))
        return NULL;
    return PyLong_FromLong(mx_gemm(A, M, K, lda, P, N, C, ldc, W, wsb, S));
}

/* gemm_with_plan(A, M, K, lda, packed, N, C, ldc, ws, ws_bytes,
 *                mb, nb, wn, wk, splits, amode, finish, stream) -> rc */
static PyObject* py_gemm_with_plan(PyObject* self, PyObject* const* a, Py_ssize_t n) {
    (void)self;
    if (n != 18) {
        PyErr_SetString(PyExc_TypeError, "gemm_with_plan expects 18 arguments");
        return NULL;
    }
    void *A, *P, *C, *W, *S;
    int M, K, lda, N, ldc;
    size_t wsb;
    mx_plan plan;
    if (get_ptr(a[0], &A) || get_int(a[1], &M) || get_int(a[2], &K) || get_int(a[3], &lda) ||
        get_ptr(a[4], &P) || get_int(a[5], &N) || get_ptr(a[6], &C) || get_int(a[7], &ldc) ||
        get_ptr(a[8], &W) || get_size(a[9], &wsb) || get_int(a[10], &plan.mb) || get_int(a[11], &plan.nb) ||
        get_int(a[12], &plan.wn) || get_int(a[13], &plan.wk) || get_int(a[14], &plan.splits) ||
        get_int(a[15], &plan.amode) || get_int(a[16], &plan.finish) || get_ptr(a[17], &S))
        return NULL;
    return PyLong_FromLong(mx_gemm_with_plan(A, M, K, lda, P, N, C, ldc, W, wsb, &plan, S));
}

/* gemm_a16w4(A, M, K, lda, packed, N, C, ldc, ws, ws_bytes, stream) -> rc */
static PyObject* py_gemm_a16w4(PyObject* self, PyObject* const* a, Py_ssize_t n) {
    (void)self;
    if (n != 11) {
        PyErr_SetString(PyExc_TypeError, "gemm_a16w4 expects 11 arguments");
        return NULL;
    }
    void *A, *P, *C, *W, *S;
    int M, K, lda, N, ldc;
    size_t wsb;
    if (get_ptr(a[0], &A) || get_int(a[1], &M) || get_int(a[2], &K) || get_int(a[3], &lda) ||
        get_ptr(a[4], &P) || get_int(a[5], &N) || get_ptr(a[6], &C) || get_int(a[7], &ldc) ||
        get_ptr(a[8], &W) || get_size(a[9], &wsb) || get_ptr(a[10], &S))
        return NULL;
    return PyLong_FromLong(mx_gemm_a16w4(A, M, K, lda, P, N, C, ldc, W, wsb, S));
}

static PyMethodDef methods[] = {
    {"gemm", (PyCFunction)(void (*)(void))py_gemm, METH_FASTCALL, "mx_gemm; returns the MX_* code"},
    {"gemm_with_plan", (PyCFunction)(void (*)(void))py_gemm_with_plan, METH_FASTCALL,
     "mx_gemm_with_plan; returns the MX_* code"},
    {"gemm_a16w4", (PyCFunction)(void (*)(void))py_gemm_a16w4, METH_FASTCALL,
     "mx_gemm_a16w4; returns the MX_* code"},
    {NULL, NULL, 0, NULL},
};

static struct PyModuleDef module = {PyModuleDef_HEAD_INIT, "_mx4ext", NULL, -1, methods,
                                    NULL, NULL, NULL, NULL};

PyMODINIT_FUNC PyInit__mx4ext(void) { return PyModule_Create(&module); }
