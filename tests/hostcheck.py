"""Builds the host cache manager against the CPU stand-in backend
(tests/hostcheck_backend.cpp) for the host-logic tests.

KVC_HOSTCHECK_FLAGS (environment, space-separated) adds compiler flags: the
sanitizer run of these tests sets it, together with the sanitizer runtime.
"""
import ctypes as C
import os
import shlex
import subprocess

from incremental_kv_cache_amd import capi

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def build(tmp_path_factory, name: str):
    out = str(tmp_path_factory.mktemp(name) / "libkvc_hostcheck.so")
    extra = shlex.split(os.environ.get("KVC_HOSTCHECK_FLAGS", ""))
    cmd = ["g++", "-O1", "-g", "-std=c++17", "-fPIC", "-shared", "-Wall", "-Wextra", *extra,
           "-I", os.path.join(ROOT, "include"), "-I", os.path.join(ROOT, "incremental_kv_cache_amd", "csrc"),
           os.path.join(ROOT, "incremental_kv_cache_amd", "csrc", "kvc_host.cpp"),
           os.path.join(ROOT, "tests", "hostcheck_backend.cpp"), "-o", out]
    subprocess.run(cmd, check=True)
    return capi.declare(C.CDLL(out))
